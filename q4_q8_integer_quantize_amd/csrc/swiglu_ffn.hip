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
#include "xrow_quant.h"

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
  // NORM: x is the fp32 hidden state xf[hidden] with RMSNorm weights gamma,
  // normed and quantized by every workgroup (xq unused)
  const float* xf;
  const float* gamma;
  float eps;
};

// Wave w of WPB owns rows RPW*w .. RPW*w + RPW-1 of the block (RPW = 32 /
// WPB).  Its work is G = 2 * (RPW / (RW*R)) row groups -- gate and up
// alternating -- unrolled into straight-line code with P groups requested
// ahead, as in q4k_q8_gemv_kernel: no load sits under a branch, so each wait
// is for exactly the tile about to be reduced.  XL: the workgroup copies x
// into LDS once and the lanes read their slots from there.
template <int TPR, int S, int R, int P, int WPB = 4, bool XL = false, bool NORM = false>
__global__ __launch_bounds__(64 * WPB) void swiglu_gate_up_kernel(SwiArgs a) {
  static_assert(!NORM || (WPB == 4 && !XL), "the RMSNorm prologue runs on 256 threads");
  constexpr int RW = 8 / TPR;
  constexpr int kGroupRows = RW * R;                 // rows of one matrix per group
  constexpr int RPW = 32 / WPB;                      // rows of the block a wave owns
  static_assert(32 % WPB == 0 && RPW % kGroupRows == 0, "a wave's rows split into whole groups");
  constexpr int G = 2 * (RPW / kGroupRows);          // gate, up, gate, up, ...
  __shared__ float gs[32], us[32], hs[32];
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t blk_row0 = blockIdx.x * 32u;
  const uint32_t row0 = blk_row0 + wave * (uint32_t)RPW;
  const LaneRole ro = make_role<TPR>();
  const uint32_t row_bytes = (uint32_t)a.nsb * kQ4KBytes;
  const uint32_t bytes = (uint32_t)a.inter * row_bytes;
  const WSrc sg = make_wsrc(a.wg, row_bytes, bytes);
  const WSrc su = make_wsrc(a.wu, row_bytes, bytes);
  const LaneOffsets<TPR, S> off = lane_offsets<TPR, S>(sg, 0, ro);

  // activation first: vector loads retire in order
  XSlots<S, 1> xs;
  XStage<TPR, S, 1, WPB> xst;
  __shared__ __attribute__((aligned(16)))
  uint8_t x_lds[(XL || NORM) ? XStage<TPR, S, 1, WPB>::kLdsBytes : 16];
  constexpr int kRowPasses = (S * TPR * 8 + kXrowBlocksPerPass - 1) / kXrowBlocksPerPass;
  XRow<NORM ? kRowPasses : 1, true> xrow;
  const int hidden = a.nsb * kQKK;
  if constexpr (NORM)
    xrow_request<kRowPasses, true, true>(xrow, a.xf, a.gamma, hidden, a.nsb * 8);
  else if constexpr (XL)
    x_stage_request(xst, a.xq, (uint32_t)a.nsb * 8u * kQ8Bytes, 0, a.nsb, 1);
  else
    load_x_slots<TPR, S, 1>(xs, a.xq, 0, a.nsb, 1, ro);
  WTile<S, R> t[G];
#pragma unroll
  for (int k = 0; k < P && k < G; ++k)
    load_w_tile<TPR, S, R>(t[k], (k & 1) ? su : sg, off, row0 + (uint32_t)(k >> 1) * kGroupRows);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NORM) {
    __shared__ float part[kXrowThreads / kWave];
    xrow_quantize<kRowPasses, true, S * TPR * 8>(xrow, a.eps, hidden, a.nsb * 8, x_lds, nullptr,
                                                 part);
    // LDS-only release/acquire: the weight loads stay in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    load_x_slots_from_lds<TPR, S, 1, true>(xs, x_lds, 0u, a.nsb, 1, ro);
  } else if constexpr (XL) {
    x_stage_commit(xst, x_lds, xs, a.nsb, 1, ro);
  }
#pragma unroll
  for (int k = 0; k < G; ++k) {
    if (k + P < G)
      load_w_tile<TPR, S, R>(t[k + P], ((k + P) & 1) ? su : sg, off,
                             row0 + (uint32_t)((k + P) >> 1) * kGroupRows);
    __builtin_amdgcn_sched_barrier(0);
    float acc[R][1];
    q4k_tile_dot<TPR, S, R, 1>(acc, t[k], xs, ro);
    if (row_leader<TPR>(ro)) {
      float* dst = (k & 1) ? us : gs;
#pragma unroll
      for (int r = 0; r < R; ++r)
        dst[wave * (uint32_t)RPW + (uint32_t)(k >> 1) * kGroupRows + r * RW + ro.rs] = acc[r][0];
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

template <int TPR, int S, bool NORM>
static hipError_t run_gate_up(const SwiArgs& a, hipStream_t st) {
  constexpr int RW = 8 / TPR;
  constexpr int R_reg = S <= 2 ? 2 : 1;               // rows unrolled per group
  constexpr int R = RW * R_reg <= 8 ? R_reg : 1;
  constexpr int G = 2 * (8 / (RW * R));
  constexpr int P = G > 2 ? 2 : G - 1 > 0 ? G - 1 : 1;
  // x staged in LDS for rows of two or more slots, as in the GEMV (4096 ->
  // 2 x 14336: 13.0-13.2 against 13.2-13.4 us); more waves a workgroup
  // (8 or 16, fewer rows each) measured slower (14.3-14.8 us)
  constexpr bool XL = S >= 2 && !NORM;
  hipLaunchKernelGGL((swiglu_gate_up_kernel<TPR, S, R, P, 4, XL, NORM>), dim3(a.inter / 32),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

template <bool NORM>
static hipError_t gate_up(const SwiArgs& a, hipStream_t stream) {
  const int nsb = a.nsb;
  if (nsb == 1) return run_gate_up<1, 1, NORM>(a, stream);
  if (nsb == 2) return run_gate_up<2, 1, NORM>(a, stream);
  if (nsb <= 4) return run_gate_up<4, 1, NORM>(a, stream);
  switch ((nsb + 7) / 8) {
    case 1: return run_gate_up<8, 1, NORM>(a, stream);
    case 2: return run_gate_up<8, 2, NORM>(a, stream);
    case 3: return run_gate_up<8, 3, NORM>(a, stream);
    case 4: return run_gate_up<8, 4, NORM>(a, stream);
    case 5: return run_gate_up<8, 5, NORM>(a, stream);
    case 6: return run_gate_up<8, 6, NORM>(a, stream);
    case 7: return run_gate_up<8, 7, NORM>(a, stream);
    case 8: return run_gate_up<8, 8, NORM>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_swiglu_ffn_q4k(const uint8_t* w_gate, const uint8_t* w_up,
                                 const uint8_t* w_down, const uint8_t* xq, float* h,
                                 uint8_t* h_q8, float* y, float* gu, int hidden_dim,
                                 int inter_dim, hipStream_t stream, const float* r) {
  SwiArgs a;
  a.wg = w_gate;
  a.wu = w_up;
  a.xq = xq;
  a.h = h;
  a.hq = h_q8;
  a.gu = gu;
  a.inter = inter_dim;
  a.nsb = hidden_dim / kQKK;
  a.xf = nullptr;
  a.gamma = nullptr;
  a.eps = 0.0f;
  const hipError_t e = gate_up<false>(a, stream);
  if (e != hipSuccess) return e;
  return launch_q4k_q8_gemv(w_down, h_q8, y, hidden_dim, inter_dim, 1, stream, r);
}

// The pre-norm FFN block: y = x + W_down Q8_1(silu(g) u), g, u = W_gate, W_up
// times Q8_1(RMSNorm(x)), with the RMSNorm and quantize in every gate/up
// workgroup (bit-identical to launch_rmsnorm_q8_1 then launch_swiglu_ffn_q4k
// with r = x).
hipError_t launch_rmsnorm_swiglu_ffn_q4k(const uint8_t* w_gate, const uint8_t* w_up,
                                         const uint8_t* w_down, const float* x,
                                         const float* gamma, float eps, float* h,
                                         uint8_t* h_q8, float* y, float* gu, int hidden_dim,
                                         int inter_dim, hipStream_t stream) {
  SwiArgs a;
  a.wg = w_gate;
  a.wu = w_up;
  a.xq = nullptr;
  a.h = h;
  a.hq = h_q8;
  a.gu = gu;
  a.inter = inter_dim;
  a.nsb = hidden_dim / kQKK;
  a.xf = x;
  a.gamma = gamma;
  a.eps = eps;
  const hipError_t e = gate_up<true>(a, stream);
  if (e != hipSuccess) return e;
  return launch_q4k_q8_gemv(w_down, h_q8, y, hidden_dim, inter_dim, 1, stream, x);
}

}  // namespace rz
