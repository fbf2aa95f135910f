// q4k_gemm_mfma.hip -- Q4_K x Q8_1 for a batch of up to 8 token activations
// on the matrix cores (v_mfma_i32_16x16x64_i8).
//
// Same operation as q4k_gemv.hip (realizar 0.8.5 src/cuda/executor/cached.rs,
// transformer_layer_gpu_true_dp4a, steps 3 and 6: Q4K x Q8 integer dot
// products rescaled by the block scales), for several tokens that share one
// pass over the weights.  With 8 tokens the integer part is a small dense
// contraction, and the matrix cores take it off the vector ALUs.
//
// Operands of one MFMA (lane l: n = l % 16, g = l / 16):
//   B (K = 64 x N = 16 weight rows): lane (n, g) holds 16 nibbles of row n --
//     the low (e = 0) or high (e = 1) nibbles of qs bytes 64p + 16g .. +15,
//     i.e. sub-block j = 4p + 2(g/2) + e at positions 16(g%2) .. +15.  The two
//     16-byte loads of a super-block (p = 0, 1) feed four MFMAs (p, e).
//   A (M = 16 x K = 64): row m = 2t + h is token t, half h; lane (m, g) holds
//     token t's 16 codes of the same positions when g/2 == h, else zeros, so
//   D[2t + h][n] = isum(row n, token t, sub-block 4p + 2h + e)     (exact int32)
//   D lane l, element i = D[4g + i][n]: tokens 2g, 2g+1 (i/2), halves i%2.
// The lane rescales its four sums with the row's scales and the tokens' d, s:
//   y[t][n] += d * sum_j d_x[t][j] * (sc_j * isum) - dmin * sum_j s_x[t][j] * m_j
//
// The activation chunk sits in LDS as a plain copy of the Q8_1 blocks (one
// slot per token), brought in by direct buffer-to-LDS loads; a ninth, all-zero
// slot supplies the zero half of A, so no lane selects anything per MFMA.
// KS waves split a row block's super-blocks and add their partial sums through
// LDS in a fixed order, so the result does not depend on timing.
#include "q4k_gemv.h"
#include "rz_launch.h"

namespace rz {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4_a8 __attribute__((ext_vector_type(4), aligned(8)));   // 40-byte blocks: 8-byte aligned

constexpr int kMfmaRows = 16;     // weight rows per block (N of the MFMA)
constexpr int kMfmaTokens = 8;    // token slots (M = 8 tokens x 2 halves)
constexpr int kMfmaChunkSb = 16;  // super-blocks per column chunk
constexpr int kSbQ8Bytes = 8 * kQ8Bytes;   // Q8_1 bytes of one token per super-block (320)

// Weights of one super-block of the lane's row: qs bytes 16g .. 16g+15 and
// 64 + 16g .. 64+16g+15, and the 16-byte header.
struct MfmaTile {
  u32x4 q[2];
  u32x4 hd;
};

__device__ __forceinline__ void load_mfma_tile(MfmaTile& t, const WSrc& src, uint32_t row_off,
                                               uint32_t sb, uint32_t g) {
  const uint32_t base = row_off + sb * kQ4KBytes;
  t.q[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src.rsrc, base + 16u + 16u * g, 0, 0));
  t.q[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src.rsrc, base + 80u + 16u * g, 0, 0));
  t.hd = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src.rsrc, base, 0, 0));
}

// The sixteen 6-bit fields of a header as bytes: sc[0..3], sc[4..7], m[0..3],
// m[4..7] (same packing as the per-field decode of q4k_tile_dot).
struct Q4KScales {
  uint32_t sc_lo, sc_hi, m_lo, m_hi;
};

__device__ __forceinline__ Q4KScales q4k_scales_bytes(const u32x4& H) {
  const uint32_t hy = H.y, hz = H.z, hw = H.w;
  Q4KScales s;
  s.sc_lo = hy & 0x3F3F3F3Fu;
  s.m_lo = hz & 0x3F3F3F3Fu;
  s.sc_hi = (hw & 0x0F0F0F0Fu) | ((hy >> 2) & 0x30303030u);
  s.m_hi = ((hw >> 4) & 0x0F0F0F0Fu) | ((hz >> 2) & 0x30303030u);
  return s;
}

__device__ __forceinline__ uint32_t byte_of(uint32_t v, int k) { return (v >> (8 * k)) & 0xffu; }

// NSB: super-blocks in the column chunk (capacity); KS: waves per row block;
// P: super-blocks requested ahead.
template <int NSB, int KS, int P, bool ACC>
__global__ __launch_bounds__(256) void q4k_q8_gemm_mfma_kernel(Q4KGemvArgs a) {
  constexpr int NS = NSB / KS;            // super-blocks per wave
  constexpr int kBlocksPerWg = 4 / KS;    // row blocks per workgroup
  // LDS bytes of one token's chunk, whole 1 KiB DMA transfers
  constexpr uint32_t kSlot = (NSB * kSbQ8Bytes + 1023) / 1024 * 1024;
  constexpr int kDmaPerSlot = (int)(kSlot / 1024);
  // slot stride: 16 bytes more than the slot, so that the eight tokens' slots
  // start in different LDS banks (the A reads of one lane group hit one offset
  // in every slot)
  constexpr uint32_t kSlotStride = kSlot + 16;
  static_assert(NSB % KS == 0 && 4 % KS == 0, "split");
  __shared__ __attribute__((aligned(16))) uint8_t xs_lds[(kMfmaTokens + 1) * kSlotStride];
  __shared__ __attribute__((aligned(16))) float red[KS > 1 ? 4 * 64 * 2 : 2];

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t n = lane & 15u, g = lane >> 4;

  // (1) activation chunk -> LDS: slot t holds token t's blocks sb0*8 ..
  // (sb0+nsb)*8 - 1; tokens past n_tokens, blocks past the chunk and slot 8
  // read past the buffer and come in as zeros.  Wave w fills slots w, w+4
  // (and wave 0 the zero slot).
  const uint32_t tok_stride = (uint32_t)a.nsb_row * kSbQ8Bytes;
  const uint32_t chunk0 = (uint32_t)a.sb0 * kSbQ8Bytes;
  const uint32_t chunk_bytes = (uint32_t)a.nsb * kSbQ8Bytes;
  const uint32_t xbytes = (uint32_t)a.n_tokens * tok_stride;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.xq, (short)0, (int)xbytes, kBufferWord3);
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const uint32_t t = wave + 4u * s;     // wave-uniform
    if (t > kMfmaTokens) break;
#pragma unroll
    for (int i = 0; i < kDmaPerSlot; ++i) {
      const uint32_t b = (uint32_t)i * 1024u + 16u * lane;
      const bool on = t < (uint32_t)a.n_tokens && b < chunk_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (__attribute__((address_space(3))) void*)(xs_lds + t * kSlotStride + (uint32_t)i * 1024u), 16,
          on ? t * tok_stride + chunk0 + b : xbytes, 0, 0, 0);
    }
  }
  asm volatile("" ::: "memory");

  // (2) the first weight super-blocks of this wave's row block
  const uint32_t rb = blockIdx.x * (uint32_t)kBlocksPerWg + wave / KS;
  const uint32_t kpart = wave % KS;
  const uint32_t row_bytes = (uint32_t)a.nsb_row * kQ4KBytes;
  const WSrc src = make_wsrc(a.w, row_bytes, (uint32_t)a.out_dim * row_bytes);
  const uint32_t row_off = (rb * kMfmaRows + n) * row_bytes;
  const uint32_t sbw0 = (uint32_t)a.sb0 + kpart * NS;   // first global super-block of the wave
  MfmaTile tl[NS];
#pragma unroll
  for (int k = 0; k < P && k < NS; ++k) load_mfma_tile(tl[k], src, row_off, sbw0 + k, g);
  // every wave's activation loads have landed in LDS before any wave reads
  // them: wait for all but the 3 * min(P, NS) weight loads issued since
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(3 * (P < NS ? P : NS)) : "memory");

  // A: lane (m = n, g) reads token t = m/2 where g/2 == m%2, else the zero slot
  const uint32_t h = n & 1u;
  const uint32_t a_tok = (g >> 1) == h ? (n >> 1) : (uint32_t)kMfmaTokens;
  const uint32_t a_lane = a_tok * kSlotStride + 2u * h * kQ8Bytes + 8u + 16u * (g & 1u);
  // (d, s) records: tokens 2g, 2g+1
  const uint32_t r_lane0 = (2u * g) * kSlotStride, r_lane1 = (2u * g + 1u) * kSlotStride;

  // The LDS operands of one super-block: the four A operands and, per MFMA,
  // the (d, s) records of tokens 2g, 2g+1 for its two sub-blocks.
  struct TileLds {
    i32x4 A[4];
    float2 R[4][4];
  };
  auto lds_reads = [&](uint32_t sbl, TileLds& L) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        L.A[2 * p + e] = *(const i32x4_a8*)(xs_lds + a_lane + (sbl * 8u + (uint32_t)(4 * p + e)) * kQ8Bytes);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        // sub-blocks of MFMA (p, e): j0 = 4p + e (half 0), j1 = 4p + 2 + e (half 1)
        const uint32_t j0 = (uint32_t)(4 * p + e), j1 = j0 + 2u;
        float2(&r)[4] = L.R[2 * p + e];
        r[0] = *(const float2*)(xs_lds + r_lane0 + (sbl * 8u + j0) * kQ8Bytes);
        r[1] = *(const float2*)(xs_lds + r_lane0 + (sbl * 8u + j1) * kQ8Bytes);
        r[2] = *(const float2*)(xs_lds + r_lane1 + (sbl * 8u + j0) * kQ8Bytes);
        r[3] = *(const float2*)(xs_lds + r_lane1 + (sbl * 8u + j1) * kQ8Bytes);
      }
  };

  float y0 = 0.0f, y1 = 0.0f;   // tokens 2g and 2g+1 of row n
  const i32x4 zero = {0, 0, 0, 0};
  // A super-block's LDS reads are all issued before its MFMAs, so that their
  // latencies overlap instead of stalling between the MFMAs (outputs
  // unchanged; 10.9-11.1 against 11.2-11.3 us at 4096 -> 14336, where the
  // reads had been interleaved with the MFMAs; issuing them one super-block
  // ahead measured no better and takes 12 more VGPRs).
  TileLds cur;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    if (k + P < NS) load_mfma_tile(tl[k + P], src, row_off, sbw0 + k + P, g);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t sbl = kpart * NS + k;   // super-block within the chunk
    lds_reads(sbl, cur);
    __builtin_amdgcn_sched_barrier(0);
    i32x4 D[4];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const u32x4 Q = tl[k].q[p];
      const uint32_t w0 = Q.x, w1 = Q.y, w2 = Q.z, w3 = Q.w;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const i32x4 B = e == 0 ? (i32x4){(int)(w0 & 0x0F0F0F0Fu), (int)(w1 & 0x0F0F0F0Fu),
                                         (int)(w2 & 0x0F0F0F0Fu), (int)(w3 & 0x0F0F0F0Fu)}
                               : (i32x4){(int)((w0 >> 4) & 0x0F0F0F0Fu), (int)((w1 >> 4) & 0x0F0F0F0Fu),
                                         (int)((w2 >> 4) & 0x0F0F0F0Fu), (int)((w3 >> 4) & 0x0F0F0F0Fu)};
        D[2 * p + e] = __builtin_amdgcn_mfma_i32_16x16x64_i8(cur.A[2 * p + e], B, zero, 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const u32x4 H = tl[k].hd;
    const uint32_t hx = H.x;
    const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(hx & 0xffffu));
    const _Float16 dmin = __builtin_bit_cast(_Float16, (uint16_t)(hx >> 16));
    const Q4KScales sc = q4k_scales_bytes(H);
    float s0 = 0.0f, s1 = 0.0f, n0 = 0.0f, n1 = 0.0f;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int q = 2 * p + e, j0 = 4 * p + e, j1 = 4 * p + 2 + e;
        const int sc0 = (int)byte_of(j0 < 4 ? sc.sc_lo : sc.sc_hi, j0 & 3);
        const int sc1 = (int)byte_of(j1 < 4 ? sc.sc_lo : sc.sc_hi, j1 & 3);
        const float fm0 = (float)byte_of(j0 < 4 ? sc.m_lo : sc.m_hi, j0 & 3);
        const float fm1 = (float)byte_of(j1 < 4 ? sc.m_lo : sc.m_hi, j1 & 3);
        const float2(&r)[4] = cur.R[q];
        const i32x4 Dq = D[q];
        s0 = fmaf(r[0].x, (float)__mul24(sc0, Dq.x), s0);
        s0 = fmaf(r[1].x, (float)__mul24(sc1, Dq.y), s0);
        s1 = fmaf(r[2].x, (float)__mul24(sc0, Dq.z), s1);
        s1 = fmaf(r[3].x, (float)__mul24(sc1, Dq.w), s1);
        n0 = fmaf(r[0].y, fm0, n0);
        n0 = fmaf(r[1].y, fm1, n0);
        n1 = fmaf(r[2].y, fm0, n1);
        n1 = fmaf(r[3].y, fm1, n1);
      }
    y0 = __builtin_fmaf((float)d, s0, y0);
    y0 = __builtin_fmaf((float)dmin, -n0, y0);
    y1 = __builtin_fmaf((float)d, s1, y1);
    y1 = __builtin_fmaf((float)dmin, -n1, y1);
  }

  // (3) add the KS partial sums of the row block in a fixed order, then store
  if constexpr (KS > 1) {
    *(float2*)(red + 2u * threadIdx.x) = make_float2(y0, y1);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (kpart != 0) return;
    y0 = 0.0f;
    y1 = 0.0f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const float2 q = *(const float2*)(red + 2u * ((wave + k) * 64u + lane));
      y0 += q.x;
      y1 += q.y;
    }
  }
  // a storing chunk adds the residual (if any): y = fl(partial + r)
  const uint32_t row = rb * kMfmaRows + n;
  if (row < (uint32_t)a.out_dim) {
    const uint32_t t0 = 2u * g, t1 = 2u * g + 1u;
    if (t0 < (uint32_t)a.n_tokens) {
      const size_t i0 = (size_t)t0 * a.out_dim + row;
      float* q = a.y + i0;
      *q = ACC ? *q + y0 : (a.r ? y0 + a.r[i0] : y0);
    }
    if (t1 < (uint32_t)a.n_tokens) {
      const size_t i1 = (size_t)t1 * a.out_dim + row;
      float* q = a.y + i1;
      *q = ACC ? *q + y1 : (a.r ? y1 + a.r[i1] : y1);
    }
  }
}

template <int NSB, int KS, int P>
hipError_t launch_mfma_chunk(const Q4KGemvArgs& a, bool acc, hipStream_t st) {
  const long blocks = (a.out_dim + kMfmaRows - 1) / kMfmaRows;
  const long per_wg = 4 / KS;
  const unsigned grid = (unsigned)((blocks + per_wg - 1) / per_wg);
  if (acc)
    hipLaunchKernelGGL((q4k_q8_gemm_mfma_kernel<NSB, KS, P, true>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((q4k_q8_gemm_mfma_kernel<NSB, KS, P, false>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Column chunks of up to 16 super-blocks, accumulated into y by successive
// launches; short rows take a smaller chunk (and LDS copy).  Two waves per
// row block with two super-blocks requested ahead measured best at 4096 ->
// 14336 (deeper prefetch costs occupancy).  The access pattern -- each load
// instruction touches 16 rows -- keeps the vector L1 busy (its tag lookups
// stall the address unit): with the arithmetic replaced by a fold the kernel
// takes 9.7 us, against 6.5 us for a plain read of the same bytes.  Loads of
// whole row segments remove that stall, but every such variant built was
// slower in total (11.3-14.3 us against 11.2): the integer MFMAs and the
// rescale that consumes their sums then bound it, and this form overlaps them
// with its loads best.  Measured on this kernel itself: with the weight loads
// replaced by register values it still takes 8.6 us (the activation copy, the
// LDS reads and the rescale), and with the MFMAs replaced by a vector add 11.0
// us, no faster than with them.  Workgroups of 2, 6 and 8 waves (fewer copies
// of the activation for 8) measured 13.0, 15.4 and 11.3 us against 11.0.
hipError_t launch_q4k_q8_gemm_mfma(const uint8_t* w, const uint8_t* xq, float* y, int out_dim,
                                   int in_dim, int n_tokens, hipStream_t stream, const float* r) {
  Q4KGemvArgs a;
  a.r = r;
  a.w = w;
  a.xq = xq;
  a.y = y;
  a.out_dim = out_dim;
  a.nsb_row = in_dim / kQKK;
  a.n_tokens = n_tokens;
  for (int sb0 = 0; sb0 < a.nsb_row; sb0 += kMfmaChunkSb) {
    a.sb0 = sb0;
    a.nsb = a.nsb_row - sb0 < kMfmaChunkSb ? a.nsb_row - sb0 : kMfmaChunkSb;
    const bool acc = sb0 > 0;
    hipError_t e;
    if (a.nsb <= 4) e = launch_mfma_chunk<4, 2, 2>(a, acc, stream);
    else if (a.nsb <= 8) e = launch_mfma_chunk<8, 2, 2>(a, acc, stream);
    else e = launch_mfma_chunk<16, 2, 2>(a, acc, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rz
