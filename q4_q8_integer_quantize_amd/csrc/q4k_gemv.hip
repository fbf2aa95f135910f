// q4k_gemv.hip -- y = W x, W Q4_K, x Q8_1, 1..8 tokens sharing one weight pass.
//
// realizar 0.8.5 src/cuda/executor/cached.rs, transformer_layer_gpu_true_dp4a,
// steps 3 and 6 (q4k_q8_gemv_async(weight, q8_activation, out_dim, in_dim)).
// The token batch streams the weights once and reuses each loaded super-block
// for every token (the weights are the only large operand).
//
// From kMfmaMinTokens tokens on, the batch runs on the matrix cores
// (q4k_gemm_mfma.hip).
//
// With a residual r, the first column chunk stores fl(partial + r) and later
// chunks accumulate as without it; for one chunk y = fl(W x + r) exactly.
// r may be y itself: each element is read and written by the same lane.
//
// Work split: a group is RW*R consecutive rows (RW = 8/TPR side by side, R
// unrolled); each wave takes G groups strided by the wave count and keeps P
// more in flight while it reduces one.  Rows longer than the register-resident activation window
// are processed in column chunks by successive launches that accumulate into y.
#include "q4k_gemv.h"
#include "rz_launch.h"

namespace rz {

constexpr int kTilesInFlight = 2;   // P: weight tiles requested ahead of the one reduced
constexpr long kTargetWaves = 1024; // about one wave per SIMD (256 CUs x 4)

// Activation slots a lane holds in registers (10 VGPRs per slot and token);
// this kernel runs 1 or 2 tokens (more go to the matrix cores).
constexpr int kSlotsMax = 8;

// Rows unrolled per group: two for short rows of one or two tokens, else one.
template <int S, int NT>
constexpr int rows_unrolled() { return (S <= 2 && NT <= 2) ? 2 : 1; }

// How a column chunk's launch writes y.
enum class Epi { kStore, kAccumulate, kResidual };

// Activation staged in LDS once per workgroup for rows of two or more slots
// (measured: 14336 -> 4096 8.2 against 8.6 us, 4096 -> 14336 7.6 against
// 7.7 us); one-slot rows are short and skip the barrier.
template <int S>
constexpr bool x_in_lds() { return S >= 2; }

template <int TPR, int S, int NT, int G, int R = rows_unrolled<S, NT>()>
static hipError_t launch_g(const Q4KGemvArgs& a, long groups, Epi epi, hipStream_t st) {
  constexpr int P = G > kTilesInFlight ? kTilesInFlight : (G > 1 ? G - 1 : 1);
  constexpr bool XL = x_in_lds<S>();
  const size_t lds = XL ? XStage<TPR, S, NT, 4>::kLdsBytes : 0;
  const long waves = (groups + G - 1) / G;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  if (epi == Epi::kAccumulate)
    hipLaunchKernelGGL((q4k_q8_gemv_kernel<TPR, S, R, NT, G, P, true, 4, true, false, XL>),
                       dim3(grid), dim3(256), lds, st, a);
  else if (epi == Epi::kResidual)
    hipLaunchKernelGGL((q4k_q8_gemv_kernel<TPR, S, R, NT, G, P, false, 4, true, true, XL>),
                       dim3(grid), dim3(256), lds, st, a);
  else
    hipLaunchKernelGGL((q4k_q8_gemv_kernel<TPR, S, R, NT, G, P, false, 4, true, false, XL>),
                       dim3(grid), dim3(256), lds, st, a);
  return hipGetLastError();
}

// G (row groups per wave) is the smallest power of two, at most 8, that keeps
// the grid within a target wave count.  With the activation staged in LDS
// (two or more slots) a wave's start is cheap, and many waves in flight
// stream best: two-slot rows take one group a wave (4096 -> 14336: 7.2
// against 7.5 us at 8 groups; two tokens 9.3-9.9 against 9.8-10.2 us); rows
// of three or more slots, whose waves hold many more registers, aim at 2048
// waves (14336 -> 4096: 7.7-7.9 us at 2 groups, 8.2 at 4, 8.1-8.4 at 1).
// One-slot rows read x directly and aim at about one wave per SIMD.
template <int S>
constexpr long target_waves() { return S >= 3 ? 2048 : kTargetWaves; }

template <int TPR, int S, int NT>
static hipError_t run_q4k(const Q4KGemvArgs& a, Epi epi, hipStream_t st) {
  // Short two-slot matrices of one token take one row a group, so that the
  // grid still reaches every CU: 1024 x 4096 (a K or V projection) 2.78 us
  // against 2.91 us with two rows (outputs bit-identical; 4096 rows and more
  // gain nothing, 14336 rows lose 0.2-0.4 us).
  if constexpr (S == 2 && NT == 1 && TPR == 8) {
    if (a.out_dim < 2048) return launch_g<TPR, S, NT, 1, 1>(a, a.out_dim, epi, st);
  }
  constexpr int R = rows_unrolled<S, NT>();
  constexpr int RW = 8 / TPR;
  const long rows_per_group = (long)RW * R;
  const long groups = (a.out_dim + rows_per_group - 1) / rows_per_group;
  const long target = S == 2 ? groups : target_waves<S>();
  const long per_wave = (groups + target - 1) / target;
  if (per_wave <= 1) return launch_g<TPR, S, NT, 1>(a, groups, epi, st);
  if (per_wave <= 2) return launch_g<TPR, S, NT, 2>(a, groups, epi, st);
  if (per_wave <= 4) return launch_g<TPR, S, NT, 4>(a, groups, epi, st);
  return launch_g<TPR, S, NT, 8>(a, groups, epi, st);
}

template <int NT>
static hipError_t run_q4k_chunk(const Q4KGemvArgs& a, Epi epi, hipStream_t st) {
  const int nsb = a.nsb;
  if (nsb == 1) return run_q4k<1, 1, NT>(a, epi, st);
  if (nsb == 2) return run_q4k<2, 1, NT>(a, epi, st);
  if (nsb <= 4) return run_q4k<4, 1, NT>(a, epi, st);
  switch ((nsb + 7) / 8) {
    case 1: return run_q4k<8, 1, NT>(a, epi, st);
    case 2: return run_q4k<8, 2, NT>(a, epi, st);
    case 3: return run_q4k<8, 3, NT>(a, epi, st);
    case 4: return run_q4k<8, 4, NT>(a, epi, st);
    case 5: return run_q4k<8, 5, NT>(a, epi, st);
    case 6: return run_q4k<8, 6, NT>(a, epi, st);
    case 7: return run_q4k<8, 7, NT>(a, epi, st);
    case 8: return run_q4k<8, 8, NT>(a, epi, st);
    default: return hipErrorInvalidValue;
  }
}

template <int NT>
static hipError_t run_q4k_all(Q4KGemvArgs a, hipStream_t st) {
  const int chunk = 8 * kSlotsMax;
  for (int sb0 = 0; sb0 < a.nsb_row; sb0 += chunk) {
    a.sb0 = sb0;
    a.nsb = a.nsb_row - sb0 < chunk ? a.nsb_row - sb0 : chunk;
    const Epi epi = sb0 > 0 ? Epi::kAccumulate : (a.r ? Epi::kResidual : Epi::kStore);
    const hipError_t e = run_q4k_chunk<NT>(a, epi, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_q4k_q8_gemv(const uint8_t* w, const uint8_t* xq, float* y, int out_dim,
                              int in_dim, int n_tokens, hipStream_t stream, const float* r) {
  Q4KGemvArgs a;
  a.r = r;
  a.w = w;
  a.xq = xq;
  a.y = y;
  a.out_dim = out_dim;
  a.nsb_row = in_dim / kQKK;
  a.sb0 = 0;
  a.nsb = a.nsb_row;
  a.n_tokens = n_tokens;
  if (n_tokens >= kMfmaMinTokens)
    return launch_q4k_q8_gemm_mfma(w, xq, y, out_dim, in_dim, n_tokens, stream, r);
  if (n_tokens == 1) return run_q4k_all<1>(a, stream);
  return run_q4k_all<2>(a, stream);
}

}  // namespace rz
