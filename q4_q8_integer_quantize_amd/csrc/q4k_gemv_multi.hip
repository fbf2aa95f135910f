// q4k_gemv_multi.hip -- several Q4_K matrices times one Q8_1 activation in
// one launch.
//
// realizar 0.8.5 src/cuda/executor/cached.rs, transformer_layer_gpu_true_dp4a,
// steps 2-3: the activation is quantized to Q8_1 once and the Q, K and V
// projections all read it.  Launched one by one, the small K and V matrices
// (1024 x 4096 in a 7B-class GQA layer, 2.4 MB) cost more in launch and ramp
// than in streaming.  Here the row groups of all matrices form one grid: wave
// w takes groups w, w+W, ..., and finds each group's matrix in a prefix table
// (a scalar loop over at most 8 entries).  The per-row arithmetic is exactly
// that of q4k_q8_gemv_kernel with the same template parameters, so every y[m]
// equals a separate rz_q4k_q8_gemv call bit for bit.
#include "q4k_gemv.h"
#include "rz_launch.h"
#include "xrow_quant.h"

namespace rz {

struct Q4KMultiArgs {
  const uint8_t* xq;
  int nsb;                          // super-blocks per row (all matrices)
  int n_tokens;
  int n_mats;
  const uint8_t* w[kMaxMats];
  float* y[kMaxMats];
  int out_dim[kMaxMats];
  uint32_t group0[kMaxMats + 1];    // first row group of each matrix; [n_mats] = total
  // NORM: the activation is the fp32 row xf[n] with weights gamma[n], RMSNorm'ed
  // and quantized by every workgroup (xq then unused; WG 0 writes the blocks
  // to xq_out when it is not null)
  const float* xf;
  const float* gamma;
  float eps;
  int n;
  uint8_t* xq_out;
};

// LATE (NORM only): request the weight tiles only once the row of x and gamma
// has arrived, so the row's loads do not queue behind the whole launch's
// weight stream.
template <int TPR, int S, int R, int NT, int G, int P, bool XL = false, bool NORM = false,
          bool XV = true, bool LATE = false>
__global__ __launch_bounds__(256) void q4k_q8_gemv_multi_kernel(Q4KMultiArgs a) {
  static_assert(!NORM || (NT == 1 && !XL), "the RMSNorm prologue serves one token");
  static_assert(!LATE || NORM, "LATE orders the RMSNorm prologue's loads");
  constexpr int RW = 8 / TPR;
  constexpr uint32_t kRowsPerGroup = (uint32_t)RW * R;
  const uint32_t nwaves = gridDim.x * 4u;
  const uint32_t wid = __builtin_amdgcn_readfirstlane(blockIdx.x * 4u + (threadIdx.x >> 6));
  const LaneRole ro = make_role<TPR>();
  const uint32_t row_bytes = (uint32_t)a.nsb * kQ4KBytes;

  // group k of this wave: matrix m[k] (wave-uniform), first row rb[k]; groups
  // past the end use matrix 0 at a row past its end (reads zeros, stores nothing)
  int m[G];
  uint32_t rb[G];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const uint32_t gidx = wid + (uint32_t)k * nwaves;
    int mm = 0;
    uint32_t first = 0;
#pragma unroll
    for (int j = 1; j < kMaxMats; ++j) {
      const bool in = j < a.n_mats && gidx >= a.group0[j];
      mm = in ? j : mm;
      first = in ? a.group0[j] : first;
    }
    uint32_t total = a.group0[0];
#pragma unroll
    for (int j = 1; j <= kMaxMats; ++j) total = j == a.n_mats ? a.group0[j] : total;
    const bool past = gidx >= total;
    m[k] = past ? 0 : mm;
    rb[k] = past ? (uint32_t)a.out_dim[0] : (gidx - first) * kRowsPerGroup;
  }
  // the matrix's fields by select chains (a dynamic index into the kernel
  // argument block would go through scratch memory)
  auto w_of = [&](int mm) {
    const uint8_t* p = a.w[0];
#pragma unroll
    for (int j = 1; j < kMaxMats; ++j) p = mm == j ? a.w[j] : p;
    return p;
  };
  auto y_of = [&](int mm) {
    float* p = a.y[0];
#pragma unroll
    for (int j = 1; j < kMaxMats; ++j) p = mm == j ? a.y[j] : p;
    return p;
  };
  auto rows_of = [&](int mm) {
    int r = a.out_dim[0];
#pragma unroll
    for (int j = 1; j < kMaxMats; ++j) r = mm == j ? a.out_dim[j] : r;
    return r;
  };
  auto src_of = [&](int k) {
    return make_wsrc(w_of(m[k]), row_bytes, (uint32_t)rows_of(m[k]) * row_bytes);
  };
  const LaneOffsets<TPR, S> off = lane_offsets<TPR, S>(src_of(0), 0, ro);

  // activation first (XL: staged in LDS once per workgroup, as in the GEMV;
  // NORM: the fp32 row, RMSNorm'ed and quantized into LDS by the workgroup)
  XSlots<S, NT> xs;
  XStage<TPR, S, NT, 4> xst;
  extern __shared__ __attribute__((aligned(16))) uint8_t xl_lds[];
  constexpr int kRowPasses = (S * TPR * 8 + kXrowBlocksPerPass - 1) / kXrowBlocksPerPass;
  XRow<NORM ? kRowPasses : 1, true> xrow;
  if constexpr (NORM)
    xrow_request<kRowPasses, XV, true>(xrow, a.xf, a.gamma, a.n, a.nsb * 8);
  else if constexpr (XL)
    x_stage_request(xst, a.xq, (uint32_t)a.nsb * 8u * kQ8Bytes, 0, a.nsb, a.n_tokens);
  else
    load_x_slots<TPR, S, NT>(xs, a.xq, (size_t)a.nsb * 8 * kQ8Bytes, a.nsb, a.n_tokens, ro);
  WTile<S, R> t[G];
  // only the row's loads are outstanding here
  if constexpr (LATE) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int k = 0; k < P && k < G; ++k) load_w_tile<TPR, S, R>(t[k], src_of(k), off, rb[k]);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NORM) {
    __shared__ float part[kXrowThreads / kWave];
    xrow_quantize<kRowPasses, true, S * TPR * 8>(xrow, a.eps, a.n, a.nsb * 8, xl_lds,
                                                 blockIdx.x == 0 ? a.xq_out : nullptr, part);
    // LDS-only release/acquire: the weight loads stay in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    static_assert(NT == 1, "the RMSNorm prologue serves one token");
    load_x_slots_from_lds<TPR, S, NT, true>(xs, xl_lds, 0u, a.nsb, 1, ro);
  } else if constexpr (XL) {
    x_stage_commit(xst, xl_lds, xs, a.nsb, a.n_tokens, ro);
  }
#pragma unroll
  for (int k = 0; k < G; ++k) {
    if (k + P < G) load_w_tile<TPR, S, R>(t[k + P], src_of(k + P), off, rb[k + P]);
    __builtin_amdgcn_sched_barrier(0);
    float acc[R][NT];
    q4k_tile_dot<TPR, S, R, NT>(acc, t[k], xs, ro);
    Q4KGemvArgs ga;
    ga.r = nullptr;
    ga.w = w_of(m[k]);
    ga.xq = a.xq;
    ga.y = y_of(m[k]);
    ga.out_dim = rows_of(m[k]);
    ga.nsb_row = a.nsb;
    ga.sb0 = 0;
    ga.nsb = a.nsb;
    ga.n_tokens = a.n_tokens;
    store_rows<TPR, R, NT, false>(ga, acc, (long)rb[k], ro);
  }
}

// NORM: every workgroup redoes the RMSNorm and the quantize (32 KB of x and
// gamma from L2 at in_dim 4096), so fewer workgroups pay for less of it; but
// the row groups must still spread evenly over the 256 CUs, and deeper waves
// expose more latency.  Measured at in_dim 4096 in one process (launch
// durations in us, outputs bit-identical for every G):
//   groups   G = 1    2      3      4      8
//   2048      5.78   5.60    -     6.98  10.05
//   3072      6.94   7.08   6.47   7.16  10.16
//   4096      8.10   7.25    -     7.32  10.19
//   5120      9.20   8.66   8.99  10.04  10.29
//   6144     10.42   8.80   9.27   9.93  10.37
//   8192     13.00  10.85  11.25  10.28  10.65
// The rule that picks each row's best: up to 1024 groups, one a wave; else
// the smallest G of 2, 3, 4 whose grid fills whole rounds of 256 workgroups
// (the last at least 90% full), at most three; else one group a wave up to
// 4096 groups, two while that grid is at most 768 workgroups, and eight
// beyond.  (Before this, one group a wave up to 4096 groups and eight beyond.)
// The weights are requested once the row of x and gamma has arrived (LATE),
// so the row's loads do not queue behind them (5.60 against 5.81 us at 2048
// groups; no worse elsewhere).
static int multi_norm_groups_per_wave(long groups) {
  if (groups <= 1024) return 1;
  for (int g = 2; g <= 4; ++g) {
    const long wgs = (groups + 4L * g - 1) / (4L * g);
    const long rounds = (wgs + 255) / 256;
    if (rounds <= 3 && wgs * 10 >= (rounds * 256 - 256) * 10 + 256 * 9) return g;
  }
  if (groups <= 4096) return 1;
  if ((groups + 7) / 8 <= 768) return 2;
  return 8;
}

template <int TPR, int S, int G, bool XV>
static hipError_t launch_multi_norm_g(const Q4KMultiArgs& a, hipStream_t st) {
  constexpr int R = S <= 2 ? 2 : 1;
  constexpr int P = G > 2 ? 2 : (G > 1 ? G - 1 : 1);
  const size_t lds = (size_t)S * TPR * 8 * kQ8Bytes;   // every slot, zero blocks past the row
  const long waves = ((long)a.group0[a.n_mats] + G - 1) / G;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  hipLaunchKernelGGL((q4k_q8_gemv_multi_kernel<TPR, S, R, 1, G, P, false, true, XV, true>),
                     dim3(grid), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <int TPR, int S, bool XV>
static hipError_t run_multi_norm(Q4KMultiArgs a, hipStream_t st) {
  constexpr int R = S <= 2 ? 2 : 1;
  constexpr uint32_t rows_per_group = (uint32_t)(8 / TPR) * R;
  a.group0[0] = 0;
  for (int j = 0; j < kMaxMats; ++j)
    a.group0[j + 1] = a.group0[j] + (j < a.n_mats ? ((uint32_t)a.out_dim[j] + rows_per_group - 1) /
                                                       rows_per_group
                                                 : 0u);
  switch (multi_norm_groups_per_wave(a.group0[a.n_mats])) {
    case 1: return launch_multi_norm_g<TPR, S, 1, XV>(a, st);
    case 2: return launch_multi_norm_g<TPR, S, 2, XV>(a, st);
    case 3: return launch_multi_norm_g<TPR, S, 3, XV>(a, st);
    case 4: return launch_multi_norm_g<TPR, S, 4, XV>(a, st);
    default: return launch_multi_norm_g<TPR, S, 8, XV>(a, st);
  }
}

template <int TPR, int S>
static hipError_t run_multi_norm_x(const Q4KMultiArgs& a, hipStream_t st) {
  return (a.n & 3) == 0 ? run_multi_norm<TPR, S, true>(a, st) : run_multi_norm<TPR, S, false>(a, st);
}

template <int TPR, int S, int NT, int G>
static hipError_t launch_multi_g(const Q4KMultiArgs& a, hipStream_t st) {
  constexpr int R = (S <= 2 && NT <= 2) ? 2 : 1;
  constexpr int P = G > 2 ? 2 : (G > 1 ? G - 1 : 1);
  constexpr bool XL = S >= 2;
  const size_t lds = XL ? XStage<TPR, S, NT, 4>::kLdsBytes : 0;
  const long waves = ((long)a.group0[a.n_mats] + G - 1) / G;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  hipLaunchKernelGGL((q4k_q8_gemv_multi_kernel<TPR, S, R, NT, G, P, XL>), dim3(grid), dim3(256),
                     lds, st, a);
  return hipGetLastError();
}

// Groups per wave.  Rows of two or more slots stage x in LDS and follow the
// single-matrix rule (q4k_gemv.hip): one group a wave for two slots, about
// 2048 waves beyond (the attention set, 5120 groups: 6.4 us at one group a
// wave against 7.0-7.3 us at five without the staging).  One-slot rows read x
// directly and take ceil(groups / 1024), at most 8, so that the grid is at
// most 256 workgroups, one per CU: a grid a little over 256 leaves some CUs
// two workgroups and the launch waits for them.
template <int TPR, int S, int NT>
static hipError_t run_multi(Q4KMultiArgs a, hipStream_t st) {
  constexpr int R = (S <= 2 && NT <= 2) ? 2 : 1;
  constexpr uint32_t rows_per_group = (uint32_t)(8 / TPR) * R;
  a.group0[0] = 0;
  for (int j = 0; j < kMaxMats; ++j)
    a.group0[j + 1] = a.group0[j] + (j < a.n_mats ? ((uint32_t)a.out_dim[j] + rows_per_group - 1) /
                                                       rows_per_group
                                                 : 0u);
  const long groups = a.group0[a.n_mats];
  const long target = S == 2 ? groups : (S >= 3 ? 2048 : 1024);
  switch ((groups + target - 1) / target) {
    case 0:
    case 1: return launch_multi_g<TPR, S, NT, 1>(a, st);
    case 2: return launch_multi_g<TPR, S, NT, 2>(a, st);
    case 3: return launch_multi_g<TPR, S, NT, 3>(a, st);
    case 4: return launch_multi_g<TPR, S, NT, 4>(a, st);
    case 5: return launch_multi_g<TPR, S, NT, 5>(a, st);
    case 6: return launch_multi_g<TPR, S, NT, 6>(a, st);
    case 7: return launch_multi_g<TPR, S, NT, 7>(a, st);
    default: return launch_multi_g<TPR, S, NT, 8>(a, st);
  }
}

template <int NT>
static hipError_t run_multi_nt(const Q4KMultiArgs& a, hipStream_t st) {
  const int nsb = a.nsb;
  if (nsb == 1) return run_multi<1, 1, NT>(a, st);
  if (nsb == 2) return run_multi<2, 1, NT>(a, st);
  if (nsb <= 4) return run_multi<4, 1, NT>(a, st);
  switch ((nsb + 7) / 8) {
    case 1: return run_multi<8, 1, NT>(a, st);
    case 2: return run_multi<8, 2, NT>(a, st);
    case 3: return run_multi<8, 3, NT>(a, st);
    case 4: return run_multi<8, 4, NT>(a, st);
    case 5: return run_multi<8, 5, NT>(a, st);
    case 6: return run_multi<8, 6, NT>(a, st);
    case 7: return run_multi<8, 7, NT>(a, st);
    case 8: return run_multi<8, 8, NT>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_q4k_q8_gemv_multi(int n_mats, const uint8_t* const* w, float* const* y,
                                    const int* out_dims, const uint8_t* xq, int in_dim,
                                    int n_tokens, hipStream_t stream) {
  // one launch while the activation fits the register window of one or two
  // tokens (the single-matrix path takes the same route); otherwise one call
  // per matrix
  if (n_tokens > 2 || in_dim > kMultiMaxInDim) {
    for (int j = 0; j < n_mats; ++j) {
      const hipError_t e = launch_q4k_q8_gemv(w[j], xq, y[j], out_dims[j], in_dim, n_tokens, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  Q4KMultiArgs a;
  a.xq = xq;
  a.nsb = in_dim / kQKK;
  a.n_tokens = n_tokens;
  a.n_mats = n_mats;
  for (int j = 0; j < kMaxMats; ++j) {
    a.w[j] = j < n_mats ? w[j] : w[0];
    a.y[j] = j < n_mats ? y[j] : y[0];
    a.out_dim[j] = j < n_mats ? out_dims[j] : out_dims[0];
  }
  return n_tokens == 1 ? run_multi_nt<1>(a, stream) : run_multi_nt<2>(a, stream);
}

hipError_t launch_rmsnorm_q4k_q8_gemv_multi(int n_mats, const uint8_t* const* w, float* const* y,
                                            const int* out_dims, const float* x,
                                            const float* gamma, float eps, int n,
                                            uint8_t* xq_out, int in_dim, hipStream_t stream) {
  Q4KMultiArgs a;
  a.xq = nullptr;
  a.nsb = in_dim / kQKK;
  a.n_tokens = 1;
  a.n_mats = n_mats;
  for (int j = 0; j < kMaxMats; ++j) {
    a.w[j] = j < n_mats ? w[j] : w[0];
    a.y[j] = j < n_mats ? y[j] : y[0];
    a.out_dim[j] = j < n_mats ? out_dims[j] : 0;
  }
  a.xf = x;
  a.gamma = gamma;
  a.eps = eps;
  a.n = n;
  a.xq_out = xq_out;
  const int nsb = a.nsb;
  if (nsb == 1) return run_multi_norm_x<1, 1>(a, stream);
  if (nsb == 2) return run_multi_norm_x<2, 1>(a, stream);
  if (nsb <= 4) return run_multi_norm_x<4, 1>(a, stream);
  switch ((nsb + 7) / 8) {
    case 1: return run_multi_norm_x<8, 1>(a, stream);
    case 2: return run_multi_norm_x<8, 2>(a, stream);
    case 3: return run_multi_norm_x<8, 3>(a, stream);
    case 4: return run_multi_norm_x<8, 4>(a, stream);
    case 5: return run_multi_norm_x<8, 5>(a, stream);
    case 6: return run_multi_norm_x<8, 6>(a, stream);
    case 7: return run_multi_norm_x<8, 7>(a, stream);
    case 8: return run_multi_norm_x<8, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rz
