// xrow_quant.h -- a workgroup of 256 threads turns one fp32 activation row
// into Q8_1 blocks in its LDS, optionally RMSNorm'ed first.
//
// realizar 0.8.5 src/cuda/executor/cached.rs, transformer_layer_gpu_true_dp4a,
// steps 1-2 and 8: the hidden state is RMSNorm'ed and quantized to Q8_1 once,
// and the projections read the blocks; realizar 0.8.4
// src/gpu/adapters/using.rs, rms_norm_inplace: RMS = sqrt(mean(x^2) + eps),
// each value times 1/RMS times its weight.  Here every workgroup of a GEMV
// launch does this for itself, so the projections need no separate launch.
//
// Thread tid holds values 1024p + 4 tid .. +3 of pass p -- block 32p + tid/8,
// its eighth tid%8 -- which is the layout of rmsnorm_q8_1_slice_kernel and of
// the Q8_1 block rule (q8_1_block_group8).  The sum of squares runs in the
// same order as there (one fma chain per thread over passes and values, a DPP
// tree in each wave, a fixed tree over the four wave sums), so the blocks are
// bit-identical to rz_rmsnorm_q8_1 (and, without the norm, to
// rz_q8_1_quantize).
#pragma once

#include "rz_device.h"

namespace rz {

constexpr int kXrowThreads = 256;
constexpr int kXrowBlocksPerPass = kXrowThreads / 8;   // 32 Q8_1 blocks a pass

// Sum of one value per thread over a workgroup of T threads, in a fixed order:
// a DPP tree in each wave (the sum lands in lane 63), then a tree over the
// wave sums.  `part` is LDS for T/64 floats.
template <int T>
__device__ __forceinline__ float workgroup_sum(float v, float* part) {
  constexpr int NW = T / kWave;
  v = group_sum_dpp<64>(v);
  const uint32_t tid = threadIdx.x;
  if ((tid & 63u) == 63u) part[tid >> 6] = v;
  __syncthreads();
  float w[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) w[k] = part[k];
#pragma unroll
  for (int step = 1; step < NW; step *= 2)
#pragma unroll
    for (int k = 0; k + step < NW; k += 2 * step) w[k] += w[k + step];
  return w[0];
}

// This thread's share of an activation row of n values (NP passes) and, with
// NORM, of the weights gamma.
template <int NP, bool NORM>
struct XRow {
  float x[NP][4];
  float g[NORM ? NP : 1][4];
};

// Request the thread's values; values at n and past, and blocks past nblk,
// read as 0.  XV (n % 4 == 0): one 16-byte load a pass, wholly below n or
// wholly past it; otherwise four dword loads.
template <int NP, bool XV, bool NORM>
__device__ __forceinline__ void xrow_request(XRow<NP, NORM>& r, const float* x,
                                             const float* gamma, int n, int nblk) {
  const uint32_t bytes = (uint32_t)n * 4u;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)bytes, kBufferWord3);
  // without NORM the gamma descriptor is built over x and never read
  const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(NORM ? gamma : x), (short)0, (int)bytes, kBufferWord3);
  const int qi = threadIdx.x & 7, qb = threadIdx.x >> 3;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int b = p * kXrowBlocksPerPass + qb;
    const int e = b * kQK8 + 4 * qi;
    if constexpr (XV) {
      const uint32_t off = (b < nblk && e < n) ? (uint32_t)e * 4u : bytes;
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
      const uint32_t v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
      r.x[p][0] = __builtin_bit_cast(float, v0);
      r.x[p][1] = __builtin_bit_cast(float, v1);
      r.x[p][2] = __builtin_bit_cast(float, v2);
      r.x[p][3] = __builtin_bit_cast(float, v3);
      if constexpr (NORM) {
        const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(gr, off, 0, 0));
        const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
        r.g[p][0] = __builtin_bit_cast(float, w0);
        r.g[p][1] = __builtin_bit_cast(float, w1);
        r.g[p][2] = __builtin_bit_cast(float, w2);
        r.g[p][3] = __builtin_bit_cast(float, w3);
      }
    } else {
      load_block_quad(r.x[p], xr, 0u, e, n, b < nblk, bytes);
      if constexpr (NORM) load_block_quad(r.g[p], gr, 0u, e, n, b < nblk, bytes);
    }
  }
}

// The row's nblk Q8_1 blocks into LDS at lds + 40 b (and into gout when it is
// not null), followed in LDS by zero blocks up to CAP (the blocks the copy
// holds, at most 32 NP); with NORM the values are (x * (1 / sqrt(sum x^2 / n +
// eps))) * gamma first.  `part` is LDS for 4 floats.  Ends with the block copy
// written but not yet published: the caller's barrier does that.
template <int NP, bool NORM, int CAP>
__device__ __forceinline__ void xrow_quantize(const XRow<NP, NORM>& r, float eps, int n, int nblk,
                                              uint8_t* lds, uint8_t* gout, float* part) {
  static_assert(CAP <= NP * kXrowBlocksPerPass, "the zero blocks come from the passes");
  float scale = 1.0f;
  if constexpr (NORM) {
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int k = 0; k < 4; ++k) ss = fmaf(r.x[p][k], r.x[p][k], ss);
    const float total = workgroup_sum<kXrowThreads>(ss, part);
    scale = 1.0f / sqrtf(total / (float)n + eps);
  }
  const int qi = threadIdx.x & 7, qb = threadIdx.x >> 3;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int b = p * kXrowBlocksPerPass + qb;
    // whole 8-lane groups take the same branch; past nblk the values read as
    // zeros, so the blocks quantize to zero blocks
    if (b < CAP) {
      float v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = r.x[p][k];
      if constexpr (NORM) {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (v[k] * scale) * r.g[p][k];
      }
      float d, s;
      const uint32_t packed = q8_1_block_group8(v, d, s);
      uint8_t* blk = lds + b * kQ8Bytes;
      *(uint32_t*)(blk + 8 + 4 * qi) = packed;
      if (qi == 0) {
        ((float*)blk)[0] = d;
        ((float*)blk)[1] = s;
      }
      if (gout && b < nblk) {
        uint8_t* go = gout + (size_t)b * kQ8Bytes;
        *(uint32_t*)(go + 8 + 4 * qi) = packed;
        if (qi == 0) {
          ((float*)go)[0] = d;
          ((float*)go)[1] = s;
        }
      }
    }
  }
}

}  // namespace rz
