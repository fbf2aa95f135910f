// q4k_gemv.h -- Q4_K x Q8_1 row-dot machinery shared by the GEMV kernel and
// the fused SwiGLU gate/up kernel.
//
// Integer form of the product (realizar 0.8.5 src/cuda/executor/cached.rs,
// transformer_layer_gpu_true_dp4a, steps 3 and 6: Q4K x Q8 integer dot
// product): for every 32-value sub-block j of a super-block,
//   isum_j = sum_l q4[32 j + l] * q8[32 j + l]         (exact, int32)
//   y     += d * sc_j * dx_j * isum_j - dmin * m_j * s_j   (fp32)
//
// Lane roles inside a wave (lane = 8 * team + i):
//   i (0..7)   reads the 16-byte slice i of a super-block's qs: chunk c = i/2,
//              half h = i%2, i.e. 16 low nibbles of sub-block 2c and 16 high
//              nibbles of sub-block 2c+1, both at positions 16h..16h+15.
//              After exchanging half sums with lane i^1 it owns sub-block j = i.
//   team (0..7) rs = team / TPR picks one of the RW = 8/TPR rows processed side
//              by side; tslot = team % TPR takes super-blocks sb = s*TPR + tslot
//              for slots s < S.  A row is reduced over its 8*TPR lanes.
// Each lane keeps the activation codes of its S slots in registers for the
// life of the wave, so weights are the only per-row memory traffic.
#pragma once

#include "rz_device.h"

namespace rz {

template <int S, int NT>
struct XSlots {
  int lo[NT][S][4];   // codes of sub-block 2c, positions 16h..16h+15
  int hi[NT][S][4];   // codes of sub-block 2c+1, same positions
  float dx[NT][S];    // d of sub-block j = i
  float sx[NT][S];    // s of sub-block j = i
};

struct LaneRole {
  int lane, i, c, h, rs, tslot;
  // sub-block j = i: where its 6-bit scale and min sit in the 12 scale bytes
  bool hij;
  uint32_t sh_sc, sh_m, len_lo, sh_hi, len_hi;
};

template <int TPR>
__device__ __forceinline__ LaneRole make_role() {
  LaneRole r;
  r.lane = threadIdx.x & (kWave - 1);
  r.i = r.lane & 7;
  const int team = r.lane >> 3;
  r.c = r.i >> 1;
  r.h = r.i & 1;
  r.rs = team / TPR;
  r.tslot = team % TPR;
  const int jj = r.i & 3;
  r.hij = r.i >= 4;
  // j < 4 : sc = scales[j] & 63, m = scales[j+4] & 63
  // j >= 4: sc = (scales[j+4] & 15) | (scales[j-4] >> 6) << 4
  //         m  = (scales[j+4] >> 4) | (scales[j]   >> 6) << 4
  r.sh_sc = 8u * jj;
  r.sh_m = r.hij ? 8u * jj + 4u : 8u * jj;
  r.len_lo = r.hij ? 4u : 6u;
  r.sh_hi = 8u * jj + 6u;
  r.len_hi = r.hij ? 2u : 0u;
  return r;
}

// Load the activation slots of one lane.  `xq` points at token 0, block 0 of
// the chunk; token t starts tok_stride bytes later.  Slots past `nsb` and
// tokens past `n_tokens` are zero, which makes their contributions exactly 0.
template <int TPR, int S, int NT>
__device__ __forceinline__ void load_x_slots(XSlots<S, NT>& xs, const uint8_t* __restrict__ xq,
                                             size_t tok_stride, int nsb, int n_tokens,
                                             const LaneRole& ro) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int sb = s * TPR + ro.tslot;
      if (t < n_tokens && sb < nsb) {
        const uint8_t* xb = xq + (size_t)t * tok_stride + (size_t)sb * 8 * kQ8Bytes;
        const uint2* plo = (const uint2*)(xb + (2 * ro.c) * kQ8Bytes + 8 + 16 * ro.h);
        const uint2* phi = (const uint2*)(xb + (2 * ro.c + 1) * kQ8Bytes + 8 + 16 * ro.h);
        const uint2 a0 = plo[0], a1 = plo[1], b0 = phi[0], b1 = phi[1];
        xs.lo[t][s][0] = (int)a0.x; xs.lo[t][s][1] = (int)a0.y;
        xs.lo[t][s][2] = (int)a1.x; xs.lo[t][s][3] = (int)a1.y;
        xs.hi[t][s][0] = (int)b0.x; xs.hi[t][s][1] = (int)b0.y;
        xs.hi[t][s][2] = (int)b1.x; xs.hi[t][s][3] = (int)b1.y;
        const float* own = (const float*)(xb + ro.i * kQ8Bytes);
        xs.dx[t][s] = own[0];
        xs.sx[t][s] = own[1];
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) { xs.lo[t][s][k] = 0; xs.hi[t][s][k] = 0; }
        xs.dx[t][s] = 0.0f;
        xs.sx[t][s] = 0.0f;
      }
    }
  }
}

// Partial dot products of R*RW rows (RW = 8/TPR side by side, R unrolled):
// rows row_base + r*RW + rs for r < R.  Rows at or past out_dim are clamped
// to the last row (their results are discarded by the caller).  On return
// acc[r][t] holds the full row sum in every lane of the row's lane group.
template <int TPR, int S, int R, int NT>
__device__ __forceinline__ void q4k_rows(float (&acc)[R][NT], const uint8_t* __restrict__ w,
                                         size_t row_bytes, long row_base, int out_dim,
                                         int nsb, const XSlots<S, NT>& xs, const LaneRole& ro) {
  constexpr int RW = 8 / TPR;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = 0.0f;

  u32x4 hd[R][S], qs[R][S];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    long row = row_base + (long)r * RW + ro.rs;
    if (row >= out_dim) row = out_dim - 1;
    const uint8_t* wrow = w + (size_t)row * row_bytes;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      int sb = s * TPR + ro.tslot;
      if (sb >= nsb) sb = nsb - 1;   // inactive slot: its x registers are zero
      const uint8_t* p = wrow + (size_t)sb * kQ4KBytes;
      hd[r][s] = *(const u32x4*)p;
      qs[r][s] = *(const u32x4*)(p + 16 + 16 * ro.i);
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const u32x4 H = hd[r][s];
      const float d = f16_lo(H.x), dmin = f16_hi(H.x);
      const uint32_t a_sc = ro.hij ? H.w : H.y;
      const uint32_t a_m = ro.hij ? H.w : H.z;
      const uint32_t sc = bits(a_sc, ro.sh_sc, ro.len_lo) | (bits(H.y, ro.sh_hi, ro.len_hi) << 4);
      const uint32_t m = bits(a_m, ro.sh_m, ro.len_lo) | (bits(H.z, ro.sh_hi, ro.len_hi) << 4);
      const float dsc = d * (float)sc;     // exact: 11-bit mantissa times 6 bits
      const float dmm = dmin * (float)m;   // exact
      int lo[4], hi[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lo[k] = (int)(qs[r][s][k] & 0x0F0F0F0Fu);
        hi[k] = (int)((qs[r][s][k] >> 4) & 0x0F0F0F0Fu);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        int sl = 0, sh = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          sl = dot4(lo[k], xs.lo[t][s][k], sl);
          sh = dot4(hi[k], xs.hi[t][s][k], sh);
        }
        // lane h=0 keeps sub-block 2c (low nibbles), h=1 keeps 2c+1 (high);
        // each receives the partner's half sum of the sub-block it keeps
        const int keep = ro.h ? sh : sl;
        const int send = ro.h ? sl : sh;
        const int isum = keep + __shfl_xor(send, 1);
        float a = acc[r][t];
        a = fmaf(dsc, xs.dx[t][s] * (float)isum, a);
        a = fmaf(-dmm, xs.sx[t][s], a);
        acc[r][t] = a;
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = group_sum<8 * TPR>(acc[r][t]);
}

}  // namespace rz
