// q4k_gemv.h -- Q4_K x Q8_1 row-dot machinery shared by the GEMV kernel and
// the fused SwiGLU gate/up kernel.
//
// Integer form of the product (realizar 0.8.5 src/cuda/executor/cached.rs,
// transformer_layer_gpu_true_dp4a, steps 3 and 6: Q4K x Q8 integer dot
// product): for every 32-value sub-block j of a super-block,
//   isum_j = sum_l q4[32 j + l] * q8[32 j + l]                 (exact, int32)
//   y     += d * (d_x,j * (sc_j * isum_j)) - dmin * (s_j * m_j)    (fp32)
// sc_j * isum_j is an exact 24-bit integer product (|.| < 2**22).
//
// Lane roles inside a wave (lane = 8 * team + i):
//   i (0..7)   reads the 16-byte slice i of a super-block's qs: chunk c = i/2,
//              half h = i%2, i.e. 16 low nibbles of sub-block 2c and 16 high
//              nibbles of sub-block 2c+1, both at positions 16h..16h+15.  One
//              load instruction therefore covers each super-block's 128 qs
//              bytes contiguously.  After adding the partner's (lane i^1)
//              half sum the lane owns sub-block j = i.
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
  //   j < 4 : sc = scales[j] & 63, m = scales[j+4] & 63
  //   j >= 4: sc = (scales[j+4] & 15) | (scales[j-4] >> 6) << 4
  //           m  = (scales[j+4] >> 4) | (scales[j]   >> 6) << 4
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

// The same slots from a workgroup's LDS copy of the chunk's Q8_1 blocks:
// token t's blocks start at xl + t * tok_bytes.  FILLED: the copy holds every
// slot of all NT tokens, zero blocks past the chunk and past n_tokens, so the
// reads need no test (and the registers no zeroing).
template <int TPR, int S, int NT, bool FILLED = false>
__device__ __forceinline__ void load_x_slots_from_lds(XSlots<S, NT>& xs, const uint8_t* xl,
                                                      uint32_t tok_bytes, int nsb, int n_tokens,
                                                      const LaneRole& ro) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int sb = s * TPR + ro.tslot;
      if (FILLED || (t < n_tokens && sb < nsb)) {
        const uint8_t* xb = xl + t * tok_bytes + sb * 8 * kQ8Bytes;
        const uint2* plo = (const uint2*)(xb + (2 * ro.c) * kQ8Bytes + 8 + 16 * ro.h);
        const uint2* phi = (const uint2*)(xb + (2 * ro.c + 1) * kQ8Bytes + 8 + 16 * ro.h);
        const uint2 a0 = plo[0], a1 = plo[1], b0 = phi[0], b1 = phi[1];
        xs.lo[t][s][0] = (int)a0.x; xs.lo[t][s][1] = (int)a0.y;
        xs.lo[t][s][2] = (int)a1.x; xs.lo[t][s][3] = (int)a1.y;
        xs.hi[t][s][0] = (int)b0.x; xs.hi[t][s][1] = (int)b0.y;
        xs.hi[t][s][2] = (int)b1.x; xs.hi[t][s][3] = (int)b1.y;
        const float2 own = *(const float2*)(xb + ro.i * kQ8Bytes);
        xs.dx[t][s] = own.x;
        xs.sx[t][s] = own.y;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) { xs.lo[t][s][k] = 0; xs.hi[t][s][k] = 0; }
        xs.dx[t][s] = 0.0f;
        xs.sx[t][s] = 0.0f;
      }
    }
  }
}

// A workgroup's copy of the activation chunk in LDS: the chunk's Q8_1 blocks
// of every token (token t at byte t * kTokBytes), brought in 16 bytes a thread
// per step.  x_stage_request issues the loads (before the first weight
// tiles: vector loads retire in order, so waiting for them later never waits
// for a tile); x_stage_commit writes them to LDS, passes an LDS-only barrier
// (weight loads stay in flight) and fills the lane's slots from LDS.
template <int TPR, int S, int NT, int WPB>
struct XStage {
  static constexpr uint32_t kTokBytes = (uint32_t)(S * TPR * 8 * kQ8Bytes);
  static constexpr int kChunks = NT * (int)(kTokBytes / 16);
  static constexpr int kIters = (kChunks + 64 * WPB - 1) / (64 * WPB);
  static constexpr size_t kLdsBytes = (size_t)NT * kTokBytes;
  u32x4 v[kIters];
};

// xq: token 0, block 0 of the full activation; the chunk starts at super-block
// sb0 and holds nsb super-blocks; token t starts tok_stride bytes after t-1.
template <int TPR, int S, int NT, int WPB>
__device__ __forceinline__ void x_stage_request(XStage<TPR, S, NT, WPB>& st, const uint8_t* xq,
                                                uint32_t tok_stride, int sb0, int nsb,
                                                int n_tokens) {
  using X = XStage<TPR, S, NT, WPB>;
  const uint32_t chunk_bytes = (uint32_t)nsb * 8u * kQ8Bytes;
  const uint32_t xbytes = (uint32_t)n_tokens * tok_stride;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)xq, (short)0, (int)xbytes, kBufferWord3);
#pragma unroll
  for (int j = 0; j < X::kIters; ++j) {
    const uint32_t gidx = (uint32_t)(j * 64 * WPB) + threadIdx.x;
    const uint32_t tk = gidx / (X::kTokBytes / 16u), c16 = 16u * (gidx % (X::kTokBytes / 16u));
    const bool on = gidx < (uint32_t)X::kChunks && tk < (uint32_t)n_tokens && c16 < chunk_bytes;
    const uint32_t off = on ? tk * tok_stride + (uint32_t)sb0 * 8u * kQ8Bytes + c16 : xbytes;
    st.v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
  }
}

template <int TPR, int S, int NT, int WPB>
__device__ __forceinline__ void x_stage_commit(const XStage<TPR, S, NT, WPB>& st, uint8_t* lds,
                                               XSlots<S, NT>& xs, int nsb, int n_tokens,
                                               const LaneRole& ro) {
  using X = XStage<TPR, S, NT, WPB>;
#pragma unroll
  for (int j = 0; j < X::kIters; ++j) {
    const uint32_t gidx = (uint32_t)(j * 64 * WPB) + threadIdx.x;
    if (gidx < (uint32_t)X::kChunks) *(u32x4*)(lds + 16u * gidx) = st.v[j];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  // every chunk of the copy was written (zeros past the chunk and the tokens)
  load_x_slots_from_lds<TPR, S, NT, true>(xs, lds, X::kTokBytes, nsb, n_tokens, ro);
}

// Weights of R*RW rows (RW = 8/TPR side by side, R unrolled) for one lane:
// the 16-byte header and the lane's 16-byte qs slice of each slot.
template <int S, int R>
struct WTile {
  u32x4 hd[R][S];
  u32x4 qs[R][S];
};

// A weight matrix read through a raw buffer descriptor: offsets are 32-bit,
// and a read past `bytes` returns zeros instead of faulting, so rows past
// out_dim and slots past the row need no clamping (their activation
// registers are zero, or their results are never stored).
struct WSrc {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t row_bytes;
};

__device__ __forceinline__ WSrc make_wsrc(const uint8_t* w, uint32_t row_bytes, uint32_t bytes) {
  WSrc src;
  src.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, (int)bytes, kBufferWord3);
  src.row_bytes = row_bytes;
  return src;
}

// Per-lane byte offsets of a lane's header and qs slice for each slot,
// relative to the start of the lane's row: super-block sb0 + s*TPR + tslot.
template <int TPR, int S>
struct LaneOffsets {
  uint32_t hd[S];
  uint32_t qs[S];
};

template <int TPR, int S>
__device__ __forceinline__ LaneOffsets<TPR, S> lane_offsets(const WSrc& src, int sb0,
                                                            const LaneRole& ro) {
  LaneOffsets<TPR, S> o;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    o.hd[s] = (uint32_t)ro.rs * src.row_bytes + (uint32_t)(sb0 + s * TPR + ro.tslot) * kQ4KBytes;
    o.qs[s] = o.hd[s] + 16u + 16u * (uint32_t)ro.i;
  }
  return o;
}

// Rows row_base + r*RW + rs for r < R; row_base is wave-uniform.  The whole
// offset travels in the per-lane VGPR offset, which is the part the hardware
// range-checks against the descriptor (the scalar offset is not checked).
template <int TPR, int S, int R>
__device__ __forceinline__ void load_w_tile(WTile<S, R>& wt, const WSrc& src,
                                            const LaneOffsets<TPR, S>& lo, uint32_t row_base) {
  constexpr int RW = 8 / TPR;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t roff = (row_base + (uint32_t)(r * RW)) * src.row_bytes;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      wt.hd[r][s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  src.rsrc, lo.hd[s] + roff, 0, 0));
      wt.qs[r][s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  src.rsrc, lo.qs[s] + roff, 0, 0));
    }
  }
}

// Integer exchange with lane ^ 1 (DPP quad_perm [1,0,3,2]).
__device__ __forceinline__ int xor1_i(int v) { return dpp_i<0xB1>(v); }

// Multiply-accumulate one tile into acc[r][t] and reduce each row over its
// 8*TPR lanes.  On return acc[r][t] is the full row sum in the last lane of
// the row's lane group.
template <int TPR, int S, int R, int NT>
__device__ __forceinline__ void q4k_tile_dot(float (&acc)[R][NT], const WTile<S, R>& wt,
                                             const XSlots<S, NT>& xs, const LaneRole& ro) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const u32x4 H = wt.hd[r][s];
      const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(H.x & 0xffffu));
      const _Float16 dmin = __builtin_bit_cast(_Float16, (uint16_t)(H.x >> 16));
      const uint32_t a_sc = ro.hij ? H.w : H.y;
      const uint32_t a_m = ro.hij ? H.w : H.z;
      const int sc = (int)((__builtin_amdgcn_ubfe(H.y, ro.sh_hi, ro.len_hi) << 4) |
                           __builtin_amdgcn_ubfe(a_sc, ro.sh_sc, ro.len_lo));
      const int m = (int)((__builtin_amdgcn_ubfe(H.z, ro.sh_hi, ro.len_hi) << 4) |
                          __builtin_amdgcn_ubfe(a_m, ro.sh_m, ro.len_lo));
      const float fm = (float)m;
      int lo[4], hi[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lo[k] = (int)(wt.qs[r][s][k] & 0x0F0F0F0Fu);
        hi[k] = (int)((wt.qs[r][s][k] >> 4) & 0x0F0F0F0Fu);
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
        const int isum = keep + xor1_i(send);
        // the fp16 scales enter the fmas directly (v_fma_mix_f32)
        float a = acc[r][t];
        a = __builtin_fmaf((float)d, xs.dx[t][s] * (float)__mul24(sc, isum), a);
        a = __builtin_fmaf((float)dmin, -xs.sx[t][s] * fm, a);
        acc[r][t] = a;
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = group_sum_dpp<8 * TPR>(acc[r][t]);
  }
}

// True in the lane that holds a row's reduced sum.
template <int TPR>
__device__ __forceinline__ bool row_leader(const LaneRole& ro) {
  return (ro.lane & (8 * TPR - 1)) == 8 * TPR - 1;
}

struct Q4KGemvArgs {
  const uint8_t* w;   // row 0, super-block 0
  const uint8_t* xq;  // token 0, block 0
  float* y;
  int out_dim;
  int nsb_row;        // super-blocks per full row
  int sb0;            // first super-block of this column chunk
  int nsb;            // super-blocks in this chunk
  int n_tokens;
  const float* r;     // residual [n_tokens][out_dim] added by the RES store, else unused
};

// Store one tile's row sums (leader lanes only); ACC adds to y instead.
template <int TPR, int R, int NT, bool ACC>
__device__ __forceinline__ void store_rows(const Q4KGemvArgs& a, const float (&acc)[R][NT],
                                           long row_base, const LaneRole& ro) {
  constexpr int RW = 8 / TPR;
  if (!row_leader<TPR>(ro)) return;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const long row = row_base + (long)r * RW + ro.rs;
    if (row < a.out_dim) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < a.n_tokens) {
          float* dst = a.y + (size_t)t * a.out_dim + row;
          if constexpr (ACC) *dst += acc[r][t];
          else *dst = acc[r][t];
        }
      }
    }
  }
}

// The residual values of one tile's rows, [R][NT], through a buffer
// descriptor over r: rows past out_dim and tokens past n_tokens read 0.  All
// lanes of a row load the same address; only the leader uses the value.
template <int TPR, int R, int NT>
__device__ __forceinline__ void load_residual(float (&rv)[R][NT], __amdgpu_buffer_rsrc_t rr,
                                              const Q4KGemvArgs& a, long row_base,
                                              const LaneRole& ro) {
  constexpr int RW = 8 / TPR;
  const uint32_t bytes = (uint32_t)a.n_tokens * (uint32_t)a.out_dim * 4u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const long row = row_base + (long)r * RW + ro.rs;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t off = (row < a.out_dim && t < a.n_tokens)
                               ? ((uint32_t)t * (uint32_t)a.out_dim + (uint32_t)row) * 4u
                               : bytes;
      rv[r][t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, off, 0, 0));
    }
  }
}

// Store row sums plus their residual: y = fl(acc + r), one rounding.
template <int TPR, int R, int NT>
__device__ __forceinline__ void store_rows_residual(const Q4KGemvArgs& a,
                                                    const float (&acc)[R][NT],
                                                    const float (&rv)[R][NT], long row_base,
                                                    const LaneRole& ro) {
  float sum[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) sum[r][t] = acc[r][t] + rv[r][t];
  store_rows<TPR, R, NT, false>(a, sum, row_base, ro);
}

// GEMV: wave w of W takes the G row groups w, w+W, ..., w+(G-1)W (a group is
// RW*R rows).  The G groups are unrolled into straight-line code with P tiles
// in flight: group k+P is requested before group k is reduced, and because no
// load sits under a branch the compiler waits for exactly the tile it needs.
// Groups past the end read zeros through the buffer descriptor and store
// nothing.  RES (with ACC false) adds the residual a.r in the store; a group's
// residual values are requested right after its weight tile, so waiting for
// them never waits for a tile issued later.
template <int TPR, int S, int R, int NT, int G, int P, bool ACC, int WPB = 4, bool STRIDED = true,
          bool RES = false, bool XL = false>
__global__ __launch_bounds__(64 * WPB) void q4k_q8_gemv_kernel(Q4KGemvArgs a) {
  static_assert(!(RES && ACC), "the residual is added by a storing pass");
  constexpr int RW = 8 / TPR;
  constexpr uint32_t kRowsPerGroup = (uint32_t)RW * R;
  const uint32_t nwaves = gridDim.x * (uint32_t)WPB;
  const uint32_t wid = __builtin_amdgcn_readfirstlane(blockIdx.x * (uint32_t)WPB + (threadIdx.x >> 6));
  // group k of this wave: strided (wid + k*nwaves) or a contiguous band (wid*G + k)
  const uint32_t g0 = STRIDED ? wid : wid * (uint32_t)G;
  const uint32_t gstep = STRIDED ? nwaves : 1u;
  const LaneRole ro = make_role<TPR>();
  const uint32_t row_bytes = (uint32_t)a.nsb_row * kQ4KBytes;
  const WSrc src = make_wsrc(a.w, row_bytes, (uint32_t)a.out_dim * row_bytes);
  const LaneOffsets<TPR, S> off = lane_offsets<TPR, S>(src, a.sb0, ro);

  // activation first: vector loads retire in order, so waiting for x must
  // not mean waiting for weight tiles issued before it.  XL: the workgroup
  // copies the chunk's blocks into LDS once (16 bytes a thread per step) and
  // the lanes read their slots from there, instead of every wave reading
  // them from L2.
  XSlots<S, NT> xs;
  XStage<TPR, S, NT, WPB> xst;
  extern __shared__ __attribute__((aligned(16))) uint8_t xl_lds[];
  if constexpr (XL)
    x_stage_request(xst, a.xq, (uint32_t)a.nsb_row * 8u * kQ8Bytes, a.sb0, a.nsb, a.n_tokens);
  else
    load_x_slots<TPR, S, NT>(xs, a.xq + (size_t)a.sb0 * 8 * kQ8Bytes,
                             (size_t)a.nsb_row * 8 * kQ8Bytes, a.nsb, a.n_tokens, ro);
  WTile<S, R> t[G];
  float rv[G][R][NT];
  __amdgpu_buffer_rsrc_t rr;
  if constexpr (RES)
    rr = __builtin_amdgcn_make_buffer_rsrc((void*)a.r, (short)0,
                                           (int)((uint32_t)a.n_tokens * (uint32_t)a.out_dim * 4u),
                                           kBufferWord3);
#pragma unroll
  for (int k = 0; k < P && k < G; ++k) {
    load_w_tile<TPR, S, R>(t[k], src, off, (g0 + k * gstep) * kRowsPerGroup);
    if constexpr (RES)
      load_residual<TPR, R, NT>(rv[k], rr, a, (long)(g0 + k * gstep) * kRowsPerGroup, ro);
  }
  // keep the scheduler from sinking requests below the first wait
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (XL) x_stage_commit(xst, xl_lds, xs, a.nsb, a.n_tokens, ro);
#pragma unroll
  for (int k = 0; k < G; ++k) {
    if (k + P < G) {
      load_w_tile<TPR, S, R>(t[k + P], src, off, (g0 + (k + P) * gstep) * kRowsPerGroup);
      if constexpr (RES)
        load_residual<TPR, R, NT>(rv[k + P], rr, a, (long)(g0 + (k + P) * gstep) * kRowsPerGroup,
                                  ro);
    }
    __builtin_amdgcn_sched_barrier(0);
    float acc[R][NT];
    q4k_tile_dot<TPR, S, R, NT>(acc, t[k], xs, ro);
    if constexpr (RES)
      store_rows_residual<TPR, R, NT>(a, acc, rv[k], (long)(g0 + k * gstep) * kRowsPerGroup, ro);
    else
      store_rows<TPR, R, NT, ACC>(a, acc, (long)(g0 + k * gstep) * kRowsPerGroup, ro);
  }
}

}  // namespace rz
