// q4k_gemv.hip -- y = W x, W Q4_K, x Q8_1, 1..8 tokens sharing one weight pass.
//
// realizar 0.8.5 src/cuda/executor/cached.rs, transformer_layer_gpu_true_dp4a,
// steps 3 and 6 (q4k_q8_gemv_async(weight, q8_activation, out_dim, in_dim)).
// The token batch streams the weights once and reuses each loaded super-block
// for every token (the weights are the only large operand).
//
// Work split: one wave owns RW*R consecutive rows (RW = 8/TPR side by side,
// R unrolled so that R*S super-block loads per lane are in flight at once).
// Rows longer than the register-resident activation window are processed in
// column chunks by successive launches that accumulate into y.
#include "q4k_gemv.h"
#include "rz_launch.h"

namespace rz {

struct Q4KGemvArgs {
  const uint8_t* w;   // row 0, super-block 0
  const uint8_t* xq;  // token 0, block 0
  float* y;
  int out_dim;
  int nsb_row;        // super-blocks per full row
  int sb0;            // first super-block of this column chunk
  int nsb;            // super-blocks in this chunk
  int n_tokens;
  int accumulate;     // add to y instead of storing
};

template <int TPR, int S, int R, int NT>
__global__ __launch_bounds__(256) void q4k_q8_gemv_kernel(Q4KGemvArgs a) {
  constexpr int RW = 8 / TPR;
  const long wave = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long row_base = wave * (RW * R);
  if (row_base >= a.out_dim) return;   // wave-uniform
  const LaneRole ro = make_role<TPR>();
  const size_t tok_stride = (size_t)a.nsb_row * 8 * kQ8Bytes;
  XSlots<S, NT> xs;
  load_x_slots<TPR, S, NT>(xs, a.xq + (size_t)a.sb0 * 8 * kQ8Bytes, tok_stride, a.nsb,
                           a.n_tokens, ro);
  float acc[R][NT];
  q4k_rows<TPR, S, R, NT>(acc, a.w + (size_t)a.sb0 * kQ4KBytes, (size_t)a.nsb_row * kQ4KBytes,
                          row_base, a.out_dim, a.nsb, xs, ro);
  if ((ro.lane & (8 * TPR - 1)) == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const long row = row_base + (long)r * RW + ro.rs;
      if (row < a.out_dim) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < a.n_tokens) {
            float* dst = a.y + (size_t)t * a.out_dim + row;
            *dst = a.accumulate ? *dst + acc[r][t] : acc[r][t];
          }
        }
      }
    }
  }
}

// Activation slots a lane can hold in registers, per token count.
template <int NT>
constexpr int slots_max() { return NT <= 2 ? 8 : (NT == 4 ? 4 : 2); }

// Rows unrolled per wave: keep about 8 super-block loads in flight per lane
// and the register footprint bounded as tokens multiply the activation state.
template <int S, int NT>
constexpr int rows_unrolled() {
  constexpr int per = S * (NT <= 2 ? 1 : NT / 2);
  return per >= 8 ? 1 : 8 / per;
}

template <int TPR, int S, int NT>
static hipError_t run_q4k(const Q4KGemvArgs& a, hipStream_t st) {
  if constexpr (S > slots_max<NT>()) {
    return hipErrorInvalidValue;
  } else {
    constexpr int R = rows_unrolled<S, NT>();
    constexpr int RW = 8 / TPR;
    const long rows_per_wave = (long)RW * R;
    const long waves = (a.out_dim + rows_per_wave - 1) / rows_per_wave;
    const unsigned grid = (unsigned)((waves + 3) / 4);
    hipLaunchKernelGGL((q4k_q8_gemv_kernel<TPR, S, R, NT>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
  }
}

template <int NT>
static hipError_t run_q4k_chunk(const Q4KGemvArgs& a, hipStream_t st) {
  const int nsb = a.nsb;
  if (nsb == 1) return run_q4k<1, 1, NT>(a, st);
  if (nsb == 2) return run_q4k<2, 1, NT>(a, st);
  if (nsb <= 4) return run_q4k<4, 1, NT>(a, st);
  switch ((nsb + 7) / 8) {
    case 1: return run_q4k<8, 1, NT>(a, st);
    case 2: return run_q4k<8, 2, NT>(a, st);
    case 3: return run_q4k<8, 3, NT>(a, st);
    case 4: return run_q4k<8, 4, NT>(a, st);
    case 5: return run_q4k<8, 5, NT>(a, st);
    case 6: return run_q4k<8, 6, NT>(a, st);
    case 7: return run_q4k<8, 7, NT>(a, st);
    case 8: return run_q4k<8, 8, NT>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int NT>
static hipError_t run_q4k_all(Q4KGemvArgs a, hipStream_t st) {
  const int chunk = 8 * slots_max<NT>();
  for (int sb0 = 0; sb0 < a.nsb_row; sb0 += chunk) {
    a.sb0 = sb0;
    a.nsb = a.nsb_row - sb0 < chunk ? a.nsb_row - sb0 : chunk;
    a.accumulate = sb0 > 0;
    const hipError_t e = run_q4k_chunk<NT>(a, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_q4k_q8_gemv(const uint8_t* w, const uint8_t* xq, float* y, int out_dim,
                              int in_dim, int n_tokens, hipStream_t stream) {
  Q4KGemvArgs a;
  a.w = w;
  a.xq = xq;
  a.y = y;
  a.out_dim = out_dim;
  a.nsb_row = in_dim / kQKK;
  a.sb0 = 0;
  a.nsb = a.nsb_row;
  a.n_tokens = n_tokens;
  a.accumulate = 0;
  if (n_tokens == 1) return run_q4k_all<1>(a, stream);
  if (n_tokens == 2) return run_q4k_all<2>(a, stream);
  if (n_tokens <= 4) return run_q4k_all<4>(a, stream);
  return run_q4k_all<8>(a, stream);
}

}  // namespace rz
