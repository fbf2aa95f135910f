// rmsnorm_q8_1.hip -- RMSNorm of fp32 activations and their Q8_1 quantize in
// one launch.
//
// realizar 0.8.5 src/cuda/executor/cached.rs, transformer_layer_gpu_true_dp4a,
// steps 1-2 (pre-attention RMSNorm, then the Q8_1 quantize shared by Q, K and
// V) and 8 (pre-FFN RMSNorm); the RMSNorm itself as in realizar 0.8.4
// src/gpu/adapters/using.rs, rms_norm_inplace: RMS = sqrt(mean(x^2) + eps),
// then every value times 1/RMS times its weight.
//
// Rows of up to 16384 values (kSliceMaxValues): a token is split over
// ceil(n_padded / 1024) workgroups of 256 threads.  Every workgroup sums the
// squares of the whole row (the row is read from L2 once per slice, 16 KB for
// a 4096-value row) and normalizes and quantizes its own 1024-value slice; all
// of its loads are in flight at once.  Thread tid holds values 1024p + 4 tid ..
// +3 of each pass p, so an aligned group of 8 threads holds one 32-value
// block, which is the lane layout of the Q8_1 block rule (q8_1_block_group8).
// Longer rows: one 1024-thread workgroup per token, passes of 4096 values,
// and x and gamma read again for the quantize.
//
// Sum of squares: each thread runs one fma chain over its values (4 per
// pass), then a DPP tree inside each wave (6 levels) and a fixed tree over the
// wave sums (2 or 4 levels): the longest chain of dependent additions is
// 4 * ceil(n_padded / 1024) + 8 for sliced rows and 4 * ceil(n_padded / 4096)
// + 10 for longer ones, the same on every run.  The normed values are
// quantized with the rule of rz_q8_1_quantize, so the Q8_1 blocks equal
// rz_q8_1_quantize of the normed values bit for bit.
#include "rz_launch.h"
#include "xrow_quant.h"

namespace rz {

constexpr int kSliceThreads = 256;
constexpr int kSliceValues = 4 * kSliceThreads;       // 1024
constexpr int kSliceMaxValues = 16 * kSliceValues;    // 16384
constexpr int kRowThreads = 1024;
constexpr int kRowValues = 4 * kRowThreads;           // 4096

struct NormArgs {
  const float* x;
  const float* gamma;
  float eps;
  int n;
  int n_padded;
  float* normed;     // optional
  uint8_t* out;
};

// Normalize four values (x[i0 .. i0+3] of token t, in xv, with weights gv)
// and quantize their block b; the thread's 8-lane group holds the block.
__device__ __forceinline__ void quantize_quad(const NormArgs& a, uint32_t t, int b, int i0,
                                              float scale, const float (&xv)[4],
                                              const float (&gv)[4]) {
  const int nb = a.n_padded / kQK8;
  if (b >= nb) return;                               // whole 8-lane groups leave together
  float v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = (xv[k] * scale) * gv[k];
  float d, s;
  const uint32_t packed = q8_1_block_group8(v, d, s);
  const int qi = (int)(threadIdx.x & 7u);
  uint8_t* blk = a.out + ((size_t)t * nb + b) * kQ8Bytes;
  *(uint32_t*)(blk + 8 + 4 * qi) = packed;
  if (qi == 0) {
    ((float*)blk)[0] = d;
    ((float*)blk)[1] = s;
  }
  if (a.normed) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i0 + k < a.n) a.normed[(size_t)t * a.n + i0 + k] = v[k];
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, kBufferWord3);
}

// Workgroup (token t, slice sl) of a row of at most NP * 1024 values.
template <int NP>
__global__ __launch_bounds__(kSliceThreads) void rmsnorm_q8_1_slice_kernel(NormArgs a,
                                                                          int slices) {
  __shared__ float part[kSliceThreads / kWave];
  const uint32_t t = blockIdx.x / (uint32_t)slices;
  const int sl = (int)(blockIdx.x % (uint32_t)slices);
  const int tid = (int)threadIdx.x;
  const uint32_t bytes = (uint32_t)a.n * 4u;
  const __amdgpu_buffer_rsrc_t xr = row_rsrc(a.x + (size_t)t * a.n, bytes);
  const __amdgpu_buffer_rsrc_t gr = row_rsrc(a.gamma, bytes);
  const int passes = (a.n + kSliceValues - 1) / kSliceValues;
  const int i0 = sl * kSliceValues + 4 * tid;        // this thread's values of the slice

  float xs[4], gs[4], xv[NP][4];
  load_block_quad(xs, xr, 0u, i0, a.n, true, bytes);
  load_block_quad(gs, gr, 0u, i0, a.n, true, bytes);
#pragma unroll
  for (int p = 0; p < NP; ++p)
    load_block_quad(xv[p], xr, 0u, p * kSliceValues + 4 * tid, a.n, p < passes, bytes);
  float ss = 0.0f;
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int k = 0; k < 4; ++k) ss = fmaf(xv[p][k], xv[p][k], ss);
  const float total = workgroup_sum<kSliceThreads>(ss, part);
  const float scale = 1.0f / sqrtf(total / (float)a.n + a.eps);
  quantize_quad(a, t, i0 / kQK8, i0, scale, xs, gs);
}

// One workgroup per token, any row length.
__global__ __launch_bounds__(kRowThreads) void rmsnorm_q8_1_row_kernel(NormArgs a) {
  __shared__ float part[kRowThreads / kWave];
  const uint32_t t = blockIdx.x;
  const int tid = (int)threadIdx.x;
  const uint32_t bytes = (uint32_t)a.n * 4u;
  const __amdgpu_buffer_rsrc_t xr = row_rsrc(a.x + (size_t)t * a.n, bytes);
  const __amdgpu_buffer_rsrc_t gr = row_rsrc(a.gamma, bytes);
  const int passes = (a.n_padded + kRowValues - 1) / kRowValues;
  float ss = 0.0f;
  for (int p = 0; p < passes; ++p) {
    float xv[4];
    load_block_quad(xv, xr, 0u, p * kRowValues + 4 * tid, a.n, true, bytes);
#pragma unroll
    for (int k = 0; k < 4; ++k) ss = fmaf(xv[k], xv[k], ss);
  }
  const float total = workgroup_sum<kRowThreads>(ss, part);
  const float scale = 1.0f / sqrtf(total / (float)a.n + a.eps);
  for (int p = 0; p < passes; ++p) {
    const int i0 = p * kRowValues + 4 * tid;
    float xv[4], gv[4];
    load_block_quad(xv, xr, 0u, i0, a.n, true, bytes);
    load_block_quad(gv, gr, 0u, i0, a.n, true, bytes);
    quantize_quad(a, t, i0 / kQK8, i0, scale, xv, gv);
  }
}

hipError_t launch_rmsnorm_q8_1(const float* x, const float* gamma, float eps, int n,
                               int n_padded, int n_tokens, float* normed, uint8_t* x_q8,
                               hipStream_t stream) {
  const NormArgs a{x, gamma, eps, n, n_padded, normed, x_q8};
  if (n_padded > kSliceMaxValues) {
    hipLaunchKernelGGL(rmsnorm_q8_1_row_kernel, dim3(n_tokens), dim3(kRowThreads), 0, stream, a);
    return hipGetLastError();
  }
  const int slices = (n_padded + kSliceValues - 1) / kSliceValues;
  const dim3 grid((unsigned)(n_tokens * slices)), block(kSliceThreads);
  if (slices == 1) hipLaunchKernelGGL(rmsnorm_q8_1_slice_kernel<1>, grid, block, 0, stream, a, slices);
  else if (slices == 2) hipLaunchKernelGGL(rmsnorm_q8_1_slice_kernel<2>, grid, block, 0, stream, a, slices);
  else if (slices <= 4) hipLaunchKernelGGL(rmsnorm_q8_1_slice_kernel<4>, grid, block, 0, stream, a, slices);
  else if (slices <= 8) hipLaunchKernelGGL(rmsnorm_q8_1_slice_kernel<8>, grid, block, 0, stream, a, slices);
  else hipLaunchKernelGGL(rmsnorm_q8_1_slice_kernel<16>, grid, block, 0, stream, a, slices);
  return hipGetLastError();
}

}  // namespace rz
