// swiglu_ffn.hip -- SwiGLU FFN on the integer path:
//   g = W_gate x, u = W_up x, h = silu(g) * u, h_q8 = Q8_1(h), y = W_down h_q8.
//
// realizar 0.8.5 src/cuda/executor/cached.rs, transformer_layer_gpu_true_dp4a
// step 9 (fused_ffn_swiglu_gpu_true_dp4a(normed, gate, up, down, hidden,
// intermediate)); realizar 0.8.4 src/gguf/cuda/clone_layer_weights.rs,
// cuda_swiglu_ffn (SiLU on the gate output, elementwise product with the up
// output, then the down projection).
//
// Kernel 1 (swiglu_gate_up_kernel): a workgroup owns 32 consecutive
// intermediate rows -- exactly one Q8_1 block of h -- and computes those rows
// of both gate and up, so silu*up and the requantization of h run in its
// epilogue without another pass over memory.  Kernel 2 is the Q4_K x Q8_1
// GEMV of the down projection over h_q8.
#include "q4k_gemv.h"
#include "rz_launch.h"

namespace rz {

struct SwiArgs {
  const uint8_t* wg;
  const uint8_t* wu;
  const uint8_t* xq;
  float* h;
  uint8_t* hq;
  float* gu;      // optional [2][inter]
  int inter;
  int nsb;        // hidden / 256
};

template <int TPR, int S, int R>
__global__ __launch_bounds__(256) void swiglu_gate_up_kernel(SwiArgs a) {
  constexpr int RW = 8 / TPR;
  static_assert(8 % (RW * R) == 0, "a wave's 8 rows split into whole passes");
  __shared__ float gs[32], us[32], hs[32];
  const int wave = threadIdx.x >> 6;
  const long blk_row0 = (long)blockIdx.x * 32;
  const LaneRole ro = make_role<TPR>();
  XSlots<S, 1> xs;
  load_x_slots<TPR, S, 1>(xs, a.xq, 0, a.nsb, 1, ro);
  const size_t row_bytes = (size_t)a.nsb * kQ4KBytes;

#pragma unroll
  for (int mat = 0; mat < 2; ++mat) {
    const uint8_t* w = mat ? a.wu : a.wg;
    float* dst = mat ? us : gs;
#pragma unroll
    for (int r0 = 0; r0 < 8; r0 += RW * R) {
      float acc[R][1];
      const long row_base = blk_row0 + 8 * wave + r0;
      q4k_rows<TPR, S, R, 1>(acc, w, row_bytes, row_base, a.inter, a.nsb, xs, ro);
      if ((ro.lane & (8 * TPR - 1)) == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) dst[8 * wave + r0 + r * RW + ro.rs] = acc[r][0];
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 32) {
    const float g = gs[threadIdx.x], u = us[threadIdx.x];
    const float hv = g / (1.0f + expf(-g)) * u;
    hs[threadIdx.x] = hv;
    const long row = blk_row0 + threadIdx.x;
    a.h[row] = hv;
    if (a.gu) {
      a.gu[row] = g;
      a.gu[(long)a.inter + row] = u;
    }
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    const int i = threadIdx.x;
    float v[4] = {hs[4 * i], hs[4 * i + 1], hs[4 * i + 2], hs[4 * i + 3]};
    float d, s;
    const uint32_t packed = q8_1_block_group8(v, d, s);
    uint8_t* blk = a.hq + (size_t)blockIdx.x * kQ8Bytes;
    *(uint32_t*)(blk + 8 + 4 * i) = packed;
    if (i == 0) {
      ((float*)blk)[0] = d;
      ((float*)blk)[1] = s;
    }
  }
}

template <int TPR, int S>
static hipError_t run_gate_up(const SwiArgs& a, hipStream_t st) {
  constexpr int RW = 8 / TPR;
  constexpr int RMAX = 8 / RW;
  constexpr int RS = S >= 8 ? 1 : 8 / S;
  constexpr int R = RS < RMAX ? RS : RMAX;
  hipLaunchKernelGGL((swiglu_gate_up_kernel<TPR, S, R>), dim3(a.inter / 32), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_swiglu_ffn_q4k(const uint8_t* w_gate, const uint8_t* w_up,
                                 const uint8_t* w_down, const uint8_t* xq, float* h,
                                 uint8_t* h_q8, float* y, float* gu, int hidden_dim,
                                 int inter_dim, hipStream_t stream) {
  SwiArgs a;
  a.wg = w_gate;
  a.wu = w_up;
  a.xq = xq;
  a.h = h;
  a.hq = h_q8;
  a.gu = gu;
  a.inter = inter_dim;
  a.nsb = hidden_dim / kQKK;
  hipError_t e;
  const int nsb = a.nsb;
  if (nsb == 1) e = run_gate_up<1, 1>(a, stream);
  else if (nsb == 2) e = run_gate_up<2, 1>(a, stream);
  else if (nsb <= 4) e = run_gate_up<4, 1>(a, stream);
  else {
    switch ((nsb + 7) / 8) {
      case 1: e = run_gate_up<8, 1>(a, stream); break;
      case 2: e = run_gate_up<8, 2>(a, stream); break;
      case 3: e = run_gate_up<8, 3>(a, stream); break;
      case 4: e = run_gate_up<8, 4>(a, stream); break;
      case 5: e = run_gate_up<8, 5>(a, stream); break;
      case 6: e = run_gate_up<8, 6>(a, stream); break;
      case 7: e = run_gate_up<8, 7>(a, stream); break;
      case 8: e = run_gate_up<8, 8>(a, stream); break;
      default: e = hipErrorInvalidValue;
    }
  }
  if (e != hipSuccess) return e;
  return launch_q4k_q8_gemv(w_down, h_q8, y, hidden_dim, inter_dim, 1, stream);
}

}  // namespace rz
