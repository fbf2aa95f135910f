// q4_0_gemv.hip -- y = W x with W Q4_0 (the LM head) and x fp32 or Q8_1.
//
// realizar 0.8.4 src/gpu/adapters/using.rs, GpuModelQ4::forward step 5
// (q4_0_gemv_into(lm_head, normed, logits, vocab_size, hidden_dim) over the
// fp32 output of the final RMSNorm).  Weight value (q - 8) * d, value l < 16
// in the low nibble of qs[l], value 16 + l in its high nibble.
//
// A lane owns a pair of 18-byte blocks (36 bytes, 4-byte aligned when in_dim
// is a multiple of 64): block A = d | qs at bytes 0..17, block B at 18..35.
// LPR lanes share a row (RW = 64/LPR rows side by side) and a lane takes S
// pairs of it; each wave streams G row groups with P of them requested ahead.
// A Q8_1 activation stays in the lane's registers for the wave's life; an
// fp32 activation (64 values a pair) is staged once per workgroup in LDS.
//   fp32 x : sum_l q_l x_l per block, then d * (sum - 8 * sum_l x_l)
//   Q8_1 x : isum = sum_l q_l q8_l - 8 * sum_l q8_l (exact), then d * d_x * isum
//
// LM-head epilogue (EPI): the output bias is added in a store (realizar 0.8.5
// src/cuda/executor/cached.rs, preload_lm_head_bias: the bias is added to the
// logits after the LM-head GEMV), and the launch that completes the rows
// reduces them, per workgroup, to one (value, index) pair, the largest logit
// with the smallest index on ties.  argmax_merge_kernel then reduces the
// pairs, so a greedy step downloads one index instead of vocab logits
// (dispatch_lm_head_and_download brings all of them to the host).  A row that
// fits one pass gets logits = fl32(W x + bias); a longer row is summed in
// column passes, and the bias enters the first pass's store, as the residual
// does in the Q4_K GEMV: each element of a bias that is also the output is
// read before it is first written.  GELU (the GELU FFN's up projection) and
// the greedy token need the finished row and run in the last pass.
#include "rz_device.h"
#include "rz_launch.h"

namespace rz {

struct Q40Args {
  const uint8_t* w;
  const void* x;
  float* y;
  int out_dim;
  int npairs_row;   // block pairs per full row
  int p0;           // first pair of this column chunk
  int npairs;       // pairs in this chunk
  int accumulate;
  const float* bias;  // EPI: optional [out_dim] output bias (first pass only)
  float* part_val;    // EPI: optional [grid] per-workgroup best logit (last pass only)
  int* part_idx;      //      and its row
  long part_count;    // EPI with pairs: the grid the pairs were sized for
  int act;            // EPI: 1 = GELU after the bias (last pass only; the GELU FFN's up projection)
};

// Q8_1 activation slots of one lane: the codes of its S pairs (two blocks
// each), the blocks' d, and each block's code sum (for the -8 offset).
template <int S>
struct X40Q8 {
  int q[S][16];
  float dx[S][2];
  int qsum[S][2];
};

template <int LPR, int S>
__device__ __forceinline__ void load_x40_q8(X40Q8<S>& xs, const Q40Args& a, int ps) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int p = s * LPR + ps;
    const bool on = p < a.npairs;
    const long gp = (long)a.p0 + p;
    if (on) {
      const uint8_t* xb = (const uint8_t*)a.x + gp * 2 * kQ8Bytes;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint8_t* blk = xb + b * kQ8Bytes;
        xs.dx[s][b] = ((const float*)blk)[0];
        const uint2* qp = (const uint2*)(blk + 8);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint2 u = qp[k];
          xs.q[s][8 * b + 2 * k] = (int)u.x;
          xs.q[s][8 * b + 2 * k + 1] = (int)u.y;
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) xs.q[s][k] = 0;
      xs.dx[s][0] = xs.dx[s][1] = 0.0f;
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      int t = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) t = dot4(xs.q[s][8 * b + k], 0x01010101, t);
      xs.qsum[s][b] = t;
    }
  }
}

// sum_l q_l * x_l over one block; qs dwords hold values 4k..4k+3 (low
// nibbles) and 16+4k..16+4k+3 (high nibbles).  Four independent partial sums
// (one per byte position) keep the fma chains short; they are added pairwise
// at the end.
__device__ __forceinline__ float block_dot_f32(const uint32_t qs[4], const float* x) {
  // Two nibbles masked into the two halves of a dword are two fp16 denormals,
  // and v_fma_mix_f32 converts an fp16 half to fp32 inside the fma: one
  // instruction a weight where a byte conversion and an fma took two.  A low
  // nibble masked in place is exactly q * 2^-24; a high nibble masked in
  // place is 16 q * 2^-24, against its activation (values 16..31 of the
  // block) staged already scaled by 2^-4.  Every product is then exactly
  // q * x * 2^-24, every partial sum exactly 2^-24 times the one of fp32
  // weights (rounding commutes with a power-of-two scale away from
  // underflow), and accumulator b still takes byte b's low, then high nibble
  // of each dword in turn, so the result, scaled back by 2^24, equals the
  // byte-conversion sum bit for bit.
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = qs[k];
    const uint32_t w8 = w >> 8;
    const uint32_t l02 = opaque_and(w, 0x000F000Fu);     // low nibbles of bytes 0, 2
    const uint32_t h02 = opaque_and(w, 0x00F000F0u);     // high nibbles of bytes 0, 2, x16
    const uint32_t l13 = opaque_and(w8, 0x000F000Fu);    // low nibbles of bytes 1, 3
    const uint32_t h13 = opaque_and(w8, 0x00F000F0u);    // high nibbles of bytes 1, 3, x16
    acc[0] = fmaf(f16_lo(l02), x[4 * k + 0], acc[0]);
    acc[0] = fmaf(f16_lo(h02), x[16 + 4 * k + 0], acc[0]);
    acc[1] = fmaf(f16_lo(l13), x[4 * k + 1], acc[1]);
    acc[1] = fmaf(f16_lo(h13), x[16 + 4 * k + 1], acc[1]);
    acc[2] = fmaf(f16_hi(l02), x[4 * k + 2], acc[2]);
    acc[2] = fmaf(f16_hi(h02), x[16 + 4 * k + 2], acc[2]);
    acc[3] = fmaf(f16_hi(l13), x[4 * k + 3], acc[3]);
    acc[3] = fmaf(f16_hi(h13), x[16 + 4 * k + 3], acc[3]);
  }
  return ((acc[0] + acc[1]) + (acc[2] + acc[3])) * 0x1p24f;
}

__device__ __forceinline__ int block_dot_q8(const uint32_t qs[4], const int* q8) {
  int lo = 0, hi = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    lo = dot4((int)(qs[k] & 0x0F0F0F0Fu), q8[k], lo);
    hi = dot4((int)((qs[k] >> 4) & 0x0F0F0F0Fu), q8[4 + k], hi);
  }
  return lo + hi;
}

// Weights of R rows x S pair slots for one lane: the two 18-byte blocks of a
// pair as 16 + 16 + 4 bytes.  Rows past out_dim and slots past the chunk read
// row out_dim - 1 / the chunk's last pair (their results are not stored, and
// idle slots have zero activations).
template <int S, int R>
struct Q40Tile {
  u32x4_a4 v0[R][S], v1[R][S];
  uint32_t v8[R][S];
};

template <int LPR, int S, int R>
__device__ __forceinline__ void load_q40_tile(Q40Tile<S, R>& t, const Q40Args& a, long row_base,
                                              int rs, int ps, size_t row_bytes) {
  constexpr int RW = kWave / LPR;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    long row = row_base + (long)r * RW + rs;
    if (row >= a.out_dim) row = a.out_dim - 1;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      int p = s * LPR + ps;
      if (p >= a.npairs) p = a.npairs - 1;
      const uint8_t* ptr = a.w + (size_t)row * row_bytes + ((size_t)a.p0 + p) * 36;
      t.v0[r][s] = *(const u32x4_a4*)ptr;
      t.v1[r][s] = *(const u32x4_a4*)(ptr + 16);
      t.v8[r][s] = *(const uint32_t*)(ptr + 32);
    }
  }
}

// GELU, tanh form (realizar 0.8.4 src/gguf/cuda/clone_layer_weights.rs,
// cuda_gelu_ffn, for phi-2-style models), evaluated as its equal
// u * sigmoid(2 z), z = sqrt(2/pi) (u + 0.044715 u^3): for negative u this
// avoids the cancellation in 1 + tanh(z).
__device__ __forceinline__ float gelu_tanh(float u) {
  const float z2 = -1.5957691216057308f * (u + 0.044715f * (u * u * u));   // -2 z
  return u / (1.0f + expf(z2));
}

// (v, i) ranks above (bv, bi): a larger value, or an equal value at a smaller
// index.  Every pair compares, so the reduction's result is unique.
__device__ __forceinline__ bool ranks_above(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

constexpr int kNoRow = 0x7fffffff;

// Best pair over the wave, in lane 63: an inclusive scan with the ranking as
// its operator on DPP lane moves (row_shr 1, 2, 4, 8, then row_bcast 15 and
// 31); a lane without a source takes (-inf, kNoRow), which ranks below every
// pair.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void best_step(float& bv, int& bi) {
  const float ov = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, -__builtin_inff()),
                                         __builtin_bit_cast(int, bv), CTRL, ROW_MASK, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(kNoRow, bi, CTRL, ROW_MASK, 0xF, false);
  if (ranks_above(ov, oi, bv, bi)) {
    bv = ov;
    bi = oi;
  }
}

__device__ __forceinline__ void wave_best_last(float& bv, int& bi) {
  best_step<0x111, 0xF>(bv, bi);
  best_step<0x112, 0xF>(bv, bi);
  best_step<0x114, 0xF>(bv, bi);
  best_step<0x118, 0xF>(bv, bi);
  best_step<0x142, 0xA>(bv, bi);
  best_step<0x143, 0xC>(bv, bi);
}

// fp32 activation staged in LDS: pair p of the launch at byte
// p * kPairStride -- its 64 values, then the sums of its two blocks.  The 16
// bytes of padding per pair put the pairs of neighbouring lanes in different
// LDS banks.
constexpr int kPairStride = 272;

template <int S, int LPR>
constexpr size_t xl_lds_bytes() { return (size_t)S * LPR * kPairStride; }

// Wave w of W takes the G row groups w, w+W, ... (a group is RW*R rows),
// unrolled with P groups requested ahead, as in q4k_q8_gemv_kernel.
// Q8_1 x: each lane keeps the codes of its pairs in registers.  fp32 x: the
// workgroup first copies the launch's activation pairs (S*LPR of them, zeros
// past npairs) into LDS with their block sums and the lanes read them from
// there, so a lane may take many pairs of a row (64 fp32 values a pair would
// not fit in registers).
template <int LPR, int S, int R, int G, int P, bool Q8, bool ACC, bool EPI, int WPB = 4>
__global__ __launch_bounds__(64 * WPB) void q4_0_gemv_kernel(Q40Args a) {
  constexpr bool XL = !Q8;
  constexpr int RW = kWave / LPR;
  constexpr int NT = 64 * WPB;                           // threads a workgroup
  const int lane = threadIdx.x & (kWave - 1);
  const int rs = lane / LPR, ps = lane % LPR;
  const long nwaves = (long)gridDim.x * WPB;
  const long wid = __builtin_amdgcn_readfirstlane(blockIdx.x * (uint32_t)WPB + (threadIdx.x >> 6));
  const size_t row_bytes = (size_t)a.npairs_row * 36;
  extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
  constexpr int kChunks = S * LPR * 16;                  // 16-byte chunks staged
  constexpr int kIters = (kChunks + NT - 1) / NT;
  u32x4 xin[XL ? kIters : 1];
  X40Q8<Q8 ? S : 1> xs;
  if constexpr (XL) {
    // (1) request the activation: chunk g = pair g/16, values 4(g%16) .. +3
    const uint32_t xbytes = (uint32_t)a.npairs * 256u;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const float*)a.x + (size_t)a.p0 * 64), (short)0, (int)xbytes, kBufferWord3);
#pragma unroll
    for (int j = 0; j < kIters; ++j) {
      const uint32_t g = (uint32_t)(j * NT) + threadIdx.x;
      const uint32_t off = g * 16u < xbytes ? g * 16u : xbytes;
      xin[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
    }
  } else {
    load_x40_q8<LPR, S>(xs, a, ps);
  }
  // EPI: the bias of a group's rows is requested right after its weight tile
  // (a null bias reads as an empty buffer and is not added)
  const bool has_bias = EPI && a.bias != nullptr;
  const uint32_t bias_bytes = has_bias ? (uint32_t)a.out_dim * 4u : 0u;
  const __amdgpu_buffer_rsrc_t br =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.bias, (short)0, (int)bias_bytes, kBufferWord3);
  float bv[G][R];
  auto load_bias = [&](int k) {
    if constexpr (EPI) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const long row = (wid + k * nwaves) * (RW * R) + (long)r * RW + rs;
        const uint32_t off = row < a.out_dim ? (uint32_t)row * 4u : bias_bytes;
        bv[k][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(br, off, 0, 0));
      }
    }
  };
  float best_v = -__builtin_inff();
  int best_i = kNoRow;
  Q40Tile<S, R> t[G];
#pragma unroll
  for (int k = 0; k < P && k < G; ++k) {
    load_q40_tile<LPR, S, R>(t[k], a, (wid + k * nwaves) * (RW * R), rs, ps, row_bytes);
    load_bias(k);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (XL) {
    // (3) stage into LDS; eight consecutive threads hold one block and sum it
    // (vector loads retire in order: this waits for the activation only)
#pragma unroll
    for (int j = 0; j < kIters; ++j) {
      const int g = j * NT + (int)threadIdx.x;
      const u32x4 v = xin[j];
      const uint32_t v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
      const float part = (__builtin_bit_cast(float, v0) + __builtin_bit_cast(float, v1)) +
                         (__builtin_bit_cast(float, v2) + __builtin_bit_cast(float, v3));
      const float bsum = group_sum_dpp<8>(part);
      if (g < kChunks) {
        uint8_t* pair = xl + (g >> 4) * kPairStride;
        // values 16..31 of each block, the high nibbles' partners, are staged
        // scaled by 2^-4 (exact away from underflow; block_dot_f32 takes
        // those nibbles in place, as 16 q); the block sums are unscaled
        u32x4 vs = v;
        if (g & 4) {
          vs.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, v0) * 0x1p-4f);
          vs.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, v1) * 0x1p-4f);
          vs.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, v2) * 0x1p-4f);
          vs.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, v3) * 0x1p-4f);
        }
        *(u32x4*)(pair + 16 * (g & 15)) = vs;
        if ((g & 7) == 7) *(float*)(pair + 256 + 4 * ((g & 15) >> 3)) = bsum;
      }
    }
    // LDS-only release/acquire: the weight loads stay in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }
#pragma unroll
  for (int k = 0; k < G; ++k) {
    if (k + P < G) {
      load_q40_tile<LPR, S, R>(t[k + P], a, (wid + (k + P) * nwaves) * (RW * R), rs, ps, row_bytes);
      load_bias(k + P);
    }
    __builtin_amdgcn_sched_barrier(0);
    const long row_base = (wid + k * nwaves) * (RW * R);
    float ar[R];
#pragma unroll
    for (int r = 0; r < R; ++r) ar[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      // fp32 x: this slot's pair from LDS, shared by the R rows
      float xv[XL ? 64 : 1], xsum[2];
      if constexpr (XL) {
        const uint8_t* pair = xl + (s * LPR + ps) * kPairStride;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const float4 f = *(const float4*)(pair + 16 * c);
          xv[4 * c] = f.x; xv[4 * c + 1] = f.y; xv[4 * c + 2] = f.z; xv[4 * c + 3] = f.w;
        }
        const float2 sm = *(const float2*)(pair + 256);
        xsum[0] = sm.x;
        xsum[1] = sm.y;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const u32x4_a4 A = t[k].v0[r][s], B = t[k].v1[r][s];
        const float dA = f16_lo(A.x), dB = f16_hi(B.x);
        const uint32_t qa[4] = {__builtin_amdgcn_alignbyte(A.y, A.x, 2),
                                __builtin_amdgcn_alignbyte(A.z, A.y, 2),
                                __builtin_amdgcn_alignbyte(A.w, A.z, 2),
                                __builtin_amdgcn_alignbyte(B.x, A.w, 2)};
        const uint32_t qb[4] = {B.y, B.z, B.w, t[k].v8[r][s]};
        if constexpr (XL) {
          const float sa = block_dot_f32(qa, &xv[0]);
          const float sb = block_dot_f32(qb, &xv[32]);
          ar[r] = fmaf(dA, fmaf(-8.0f, xsum[0], sa), ar[r]);
          ar[r] = fmaf(dB, fmaf(-8.0f, xsum[1], sb), ar[r]);
        } else {
          const int ia = block_dot_q8(qa, &xs.q[s][0]) - 8 * xs.qsum[s][0];
          const int ib = block_dot_q8(qb, &xs.q[s][8]) - 8 * xs.qsum[s][1];
          ar[r] = fmaf(dA * xs.dx[s][0], (float)ia, ar[r]);
          ar[r] = fmaf(dB * xs.dx[s][1], (float)ib, ar[r]);
        }
      }
    }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = group_sum_dpp<LPR>(ar[r]);
    if (ps == LPR - 1) {   // the lane that holds the reduced row sum
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const long row = row_base + (long)r * RW + rs;
        if (row < a.out_dim) {
          float v = ACC ? a.y[row] + acc[r] : acc[r];
          if constexpr (EPI) {
            if (has_bias) v = v + bv[k][r];
            if (a.act) v = gelu_tanh(v);
            if (ranks_above(v, (int)row, best_v, best_i)) {
              best_v = v;
              best_i = (int)row;
            }
          }
          a.y[row] = v;
        }
      }
    }
  }
  if constexpr (EPI) {
    if (a.part_val != nullptr) {
      __shared__ float wv[WPB];
      __shared__ int wi[WPB];
      wave_best_last(best_v, best_i);
      const int wave = threadIdx.x >> 6;
      if (lane == kWave - 1) {
        wv[wave] = best_v;
        wi[wave] = best_i;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        float v = wv[0];
        int i = wi[0];
#pragma unroll
        for (int w = 1; w < WPB; ++w)
          if (ranks_above(wv[w], wi[w], v, i)) {
            v = wv[w];
            i = wi[w];
          }
        a.part_val[blockIdx.x] = v;
        a.part_idx[blockIdx.x] = i;
      }
    }
  }
}

// The best of `count` (value, index) pairs; one workgroup.  Each thread
// requests PER pairs a pass before comparing any, so a head's pairs (a few
// thousand) arrive in one round trip, and the waves reduce by DPP.  The
// ranking is a total order, so the order of the comparisons does not change
// the result.  512 threads x 5 merge the 151936-row head's 2374 pairs in
// 2.16 us against 2.81 us for 1024 threads reducing by ds_bpermute (the same
// pairs from L2, one process).
constexpr int kMergeThreads = 512, kMergePer = 5;

template <int THREADS, int PER>
__global__ __launch_bounds__(THREADS) void argmax_merge_kernel(const float* __restrict__ pv,
                                                                const int* __restrict__ pi,
                                                                int count,
                                                                int* __restrict__ out_idx,
                                                                float* __restrict__ out_val) {
  __shared__ float wv[THREADS / kWave];
  __shared__ int wi[THREADS / kWave];
  float bv = -__builtin_inff();
  int bi = kNoRow;
  for (int base = 0; base < count; base += THREADS * PER) {
    float v[PER];
    int ix[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int j = base + k * THREADS + (int)threadIdx.x;
      v[k] = j < count ? pv[j] : -__builtin_inff();
      ix[k] = j < count ? pi[j] : kNoRow;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (ranks_above(v[k], ix[k], bv, bi)) {
        bv = v[k];
        bi = ix[k];
      }
  }
  wave_best_last(bv, bi);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) {
    wv[wave] = bv;
    wi[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = wv[0];
    int i = wi[0];
#pragma unroll
    for (int w = 1; w < THREADS / kWave; ++w)
      if (ranks_above(wv[w], wi[w], v, i)) {
        v = wv[w];
        i = wi[w];
      }
    if (out_idx) *out_idx = i;
    if (out_val) *out_val = v;
  }
}

// Waves a workgroup.  Four, unless the activation staged in LDS is 128 pairs
// or more (32 KB and up): every workgroup copies it, so larger workgroups copy
// it less often, and then the count of 8, 10 or 12 whose grid gives the CUs
// the smallest even share of waves, ceil(workgroups / 256) * waves a
// workgroup (the smaller count on a tie; 16 never does better than 8 by this
// measure).  Measured, one process, outputs
// bit-identical: 160-pair rows (2560 x 10240, 2560 waves) 6.70 us at 10 (256
// workgroups) against 7.43 at 8, 7.46 at 16 and 7.81 at 4; 48-pair rows
// (10240 x 2560) 6.18 us at 4 against 6.58-6.74 at 5, 8 and 10.
template <int LPR, int S, bool Q8>
constexpr bool q40_heavy_stage() { return !Q8 && S * LPR >= 128; }

static int q40_heavy_wpb(long waves) {
  static const int kCand[] = {8, 10, 12};
  int best = 8;
  long best_share = -1;
  for (int w : kCand) {
    const long wgs = (waves + w - 1) / w;
    const long share = (wgs + 255) / 256 * w;
    if (best_share < 0 || share < best_share) {
      best = w;
      best_share = share;
    }
  }
  return best;
}

template <int LPR, int S, int R, int G, bool Q8, int WPB>
static hipError_t launch_q40_w(const Q40Args& a, long waves, bool epi, hipStream_t st) {
  constexpr int P = G > 2 ? 2 : (G > 1 ? G - 1 : 1);
  static_assert(Q8 || xl_lds_bytes<S, LPR>() <= 65536, "staged activation within 64 KiB of LDS");
  const unsigned grid = (unsigned)((waves + WPB - 1) / WPB);
  const dim3 block(64 * WPB);
  const size_t lds = Q8 ? 0 : xl_lds_bytes<S, LPR>();
  if (epi && a.part_val != nullptr && (long)grid != a.part_count) return hipErrorInvalidValue;
  if (epi) {
    if (a.accumulate)
      hipLaunchKernelGGL((q4_0_gemv_kernel<LPR, S, R, G, P, Q8, true, true, WPB>), dim3(grid), block, lds, st, a);
    else
      hipLaunchKernelGGL((q4_0_gemv_kernel<LPR, S, R, G, P, Q8, false, true, WPB>), dim3(grid), block, lds, st, a);
  } else if (a.accumulate) {
    hipLaunchKernelGGL((q4_0_gemv_kernel<LPR, S, R, G, P, Q8, true, false, WPB>), dim3(grid), block, lds, st, a);
  } else {
    hipLaunchKernelGGL((q4_0_gemv_kernel<LPR, S, R, G, P, Q8, false, false, WPB>), dim3(grid), block, lds, st, a);
  }
  return hipGetLastError();
}

template <int LPR, int S, int R, int G, bool Q8>
static hipError_t launch_q40_g(const Q40Args& a, long groups, bool epi, hipStream_t st) {
  const long waves = (groups + G - 1) / G;
  if constexpr (q40_heavy_stage<LPR, S, Q8>()) {
    switch (q40_heavy_wpb(waves)) {
      case 10: return launch_q40_w<LPR, S, R, G, Q8, 10>(a, waves, epi, st);
      case 12: return launch_q40_w<LPR, S, R, G, Q8, 12>(a, waves, epi, st);
      default: return launch_q40_w<LPR, S, R, G, Q8, 8>(a, waves, epi, st);
    }
  } else {
    return launch_q40_w<LPR, S, R, G, Q8, 4>(a, waves, epi, st);
  }
}

// Pairs a launch covers: Q8_1 x keeps up to 4 pairs a lane in registers (64
// lanes a row); fp32 x is staged in LDS, at most kXlChunkPairs pairs (60,928
// bytes, within a workgroup's 64 KiB).
constexpr int kQ8ChunkPairs = 256;
constexpr int kXlChunkPairs = 224;

// Launch shape of a column chunk of np pairs (run_q40_chunk and run_xl_chunk
// take exactly these; q4_0_lm_head_partials uses them to size the
// per-workgroup pairs).
//   Q8_1 x: LPR lanes a row up to 32 (one pair a lane), else 64 lanes and
//           ceil(np/64) pairs a lane; R = 4 / pairs rows unrolled (at least 1).
//   fp32 x: up to 16 pairs, one pair a lane and 4 rows unrolled; longer rows
//           one row a group, with 8 lanes a row up to 32 pairs, 16 up to 64,
//           32 up to 128 and 64 up to 192 (3 or 4 pairs a lane; at most a
//           third of the slots idle), and 32 lanes of 7 pairs up to 224 (64
//           lanes of 4 would need more than 64 KiB of LDS).  Measured: twice
//           the waves with a few idle slots beat every lane busy (40 pairs:
//           16 lanes x 3 at 6.4 us against 8 x 5 at 7.4 us; 160 pairs: 64 x 3
//           at 7.9 us against 32 x 5 at 8.8 us; 128 pairs: 32 x 4 at 7.1 us
//           against 16 x 8 at 8.3 us).
// Groups per wave: one, for both activation formats -- many one-group waves
// stream best (the 151936 x 1024 LM head with fp32 x, launches of the two
// shapes interleaved: 18.1 us against 20.2 us at two groups a wave).
struct Q40Shape {
  int lpr, s, r, g;
};

static int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p *= 2;
  return p;
}

static Q40Shape q40_shape(int np, bool q8) {
  Q40Shape sh;
  if (q8) {
    sh.lpr = np <= 32 ? pow2_at_least(np) : 64;
    sh.s = np <= 32 ? 1 : (np + 63) / 64;
    sh.r = sh.s >= 4 ? 1 : 4 / sh.s;
  } else if (np <= 16) {
    sh.lpr = pow2_at_least(np);
    sh.s = 1;
    sh.r = 4;
  } else {
    sh.lpr = np <= 32 ? 8 : np <= 64 ? 16 : np <= 128 ? 32 : np <= 192 ? 64 : 32;
    sh.s = (np + sh.lpr - 1) / sh.lpr;
    sh.r = 1;
  }
  sh.g = 1;
  return sh;
}

template <int LPR, int S, int R, bool Q8>
static hipError_t run_q40(const Q40Args& a, bool epi, hipStream_t st) {
  constexpr int RW = kWave / LPR;
  const long rows_per_group = (long)RW * R;
  const long groups = (a.out_dim + rows_per_group - 1) / rows_per_group;
  return launch_q40_g<LPR, S, R, 1, Q8>(a, groups, epi, st);
}

// Q8_1 activation.
static hipError_t run_q8_chunk(const Q40Args& a, bool epi, hipStream_t st) {
  const int np = a.npairs;
  if (np <= 1) return run_q40<1, 1, 4, true>(a, epi, st);
  if (np <= 2) return run_q40<2, 1, 4, true>(a, epi, st);
  if (np <= 4) return run_q40<4, 1, 4, true>(a, epi, st);
  if (np <= 8) return run_q40<8, 1, 4, true>(a, epi, st);
  if (np <= 16) return run_q40<16, 1, 4, true>(a, epi, st);
  if (np <= 32) return run_q40<32, 1, 4, true>(a, epi, st);
  switch ((np + 63) / 64) {
    case 1: return run_q40<64, 1, 4, true>(a, epi, st);
    case 2: return run_q40<64, 2, 2, true>(a, epi, st);
    case 3: return run_q40<64, 3, 1, true>(a, epi, st);
    case 4: return run_q40<64, 4, 1, true>(a, epi, st);
    default: return hipErrorInvalidValue;
  }
}

// fp32 activation, staged in LDS.
static hipError_t run_xl_chunk(const Q40Args& a, bool epi, hipStream_t st) {
  const int np = a.npairs;
  if (np <= 1) return run_q40<1, 1, 4, false>(a, epi, st);
  if (np <= 2) return run_q40<2, 1, 4, false>(a, epi, st);
  if (np <= 4) return run_q40<4, 1, 4, false>(a, epi, st);
  if (np <= 8) return run_q40<8, 1, 4, false>(a, epi, st);
  if (np <= 16) return run_q40<16, 1, 4, false>(a, epi, st);
  if (np <= 24) return run_q40<8, 3, 1, false>(a, epi, st);
  if (np <= 32) return run_q40<8, 4, 1, false>(a, epi, st);
  if (np <= 48) return run_q40<16, 3, 1, false>(a, epi, st);
  if (np <= 64) return run_q40<16, 4, 1, false>(a, epi, st);
  if (np <= 96) return run_q40<32, 3, 1, false>(a, epi, st);
  if (np <= 128) return run_q40<32, 4, 1, false>(a, epi, st);
  if (np <= 192) return run_q40<64, 3, 1, false>(a, epi, st);
  if (np <= kXlChunkPairs) return run_q40<32, 7, 1, false>(a, epi, st);
  return hipErrorInvalidValue;
}

// Column chunks.  With `epi`, the first chunk's store adds the bias and the
// last chunk's store applies GELU and collects the greedy token (one chunk
// does all three).
template <bool Q8>
static hipError_t run_q40_all(Q40Args a, bool epi, hipStream_t st) {
  const int chunk = Q8 ? kQ8ChunkPairs : kXlChunkPairs;
  const float* bias = a.bias;
  float* part_val = a.part_val;
  int* part_idx = a.part_idx;
  const int act = a.act;
  for (int p0 = 0; p0 < a.npairs_row; p0 += chunk) {
    a.p0 = p0;
    a.npairs = a.npairs_row - p0 < chunk ? a.npairs_row - p0 : chunk;
    a.accumulate = p0 > 0;
    const bool first = p0 == 0;
    const bool last = p0 + chunk >= a.npairs_row;
    a.bias = first ? bias : nullptr;
    a.act = last ? act : 0;
    a.part_val = last ? part_val : nullptr;
    a.part_idx = last ? part_idx : nullptr;
    const bool e_ = epi && (first || last);
    const hipError_t e = Q8 ? run_q8_chunk(a, e_, st) : run_xl_chunk(a, e_, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static Q40Args q40_args(const uint8_t* w, const void* x, float* y, int out_dim, int in_dim) {
  Q40Args a;
  a.w = w;
  a.x = x;
  a.y = y;
  a.out_dim = out_dim;
  a.npairs_row = in_dim / 64;
  a.p0 = 0;
  a.npairs = a.npairs_row;
  a.accumulate = 0;
  a.bias = nullptr;
  a.part_val = nullptr;
  a.part_idx = nullptr;
  a.part_count = 0;
  a.act = 0;
  return a;
}

hipError_t launch_q4_0_gemv(const uint8_t* w, const void* x, int x_format, float* y,
                            int out_dim, int in_dim, hipStream_t stream) {
  const Q40Args a = q40_args(w, x, y, out_dim, in_dim);
  return x_format == 0 ? run_q40_all<false>(a, false, stream) : run_q40_all<true>(a, false, stream);
}

long q4_0_lm_head_partials(int out_dim, int in_dim, int x_format) {
  const bool q8 = x_format == 1;
  const int npairs_row = in_dim / 64;
  const int chunk = q8 ? kQ8ChunkPairs : kXlChunkPairs;
  const int last = npairs_row - ((npairs_row - 1) / chunk) * chunk;   // pairs of the last chunk
  const Q40Shape sh = q40_shape(last, q8);
  const long rows_per_group = (long)(kWave / sh.lpr) * sh.r;
  const long groups = (out_dim + rows_per_group - 1) / rows_per_group;
  const long waves = (groups + sh.g - 1) / sh.g;
  const int wpb = (!q8 && sh.s * sh.lpr >= 128) ? q40_heavy_wpb(waves) : 4;   // launch_q40_g
  return (waves + wpb - 1) / wpb;
}

hipError_t launch_q4_0_lm_head(const uint8_t* w, const void* x, int x_format, const float* bias,
                               float* logits, int out_dim, int in_dim, int* argmax_idx,
                               float* argmax_val, float* part_val, int* part_idx,
                               hipStream_t stream) {
  Q40Args a = q40_args(w, x, logits, out_dim, in_dim);
  a.bias = bias;
  const bool argmax = argmax_idx != nullptr || argmax_val != nullptr;
  if (argmax) {
    a.part_val = part_val;
    a.part_idx = part_idx;
    a.part_count = q4_0_lm_head_partials(out_dim, in_dim, x_format);
  }
  const hipError_t e = x_format == 0 ? run_q40_all<false>(a, true, stream)
                                     : run_q40_all<true>(a, true, stream);
  if (e != hipSuccess || !argmax) return e;
  const int count = (int)q4_0_lm_head_partials(out_dim, in_dim, x_format);
  hipLaunchKernelGGL((argmax_merge_kernel<kMergeThreads, kMergePer>), dim3(1), dim3(kMergeThreads), 0,
                     stream, part_val, part_idx,
                     count, argmax_idx, argmax_val);
  return hipGetLastError();
}

// GELU FFN (realizar 0.8.4 src/gpu/adapters/using.rs, ffn_standard_gpu;
// clone_layer_weights.rs, cuda_gelu_ffn): h = gelu(W_up x + up_bias) in the
// up projection's epilogue, then y = W_down h + down_bias, both on fp32
// activations.
hipError_t launch_gelu_ffn_q4_0(const uint8_t* w_up, const uint8_t* w_down, const float* x,
                                const float* up_bias, const float* down_bias, float* h, float* y,
                                int hidden_dim, int inter_dim, hipStream_t stream) {
  Q40Args up = q40_args(w_up, x, h, inter_dim, hidden_dim);
  up.bias = up_bias;
  up.act = 1;
  hipError_t e = run_q40_all<false>(up, true, stream);
  if (e != hipSuccess) return e;
  Q40Args down = q40_args(w_down, h, y, hidden_dim, inter_dim);
  down.bias = down_bias;
  return run_q40_all<false>(down, true, stream);
}

}  // namespace rz
