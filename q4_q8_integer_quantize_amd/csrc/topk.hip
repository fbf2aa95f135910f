// topk.hip -- the k largest values of an fp32 array, largest first, equal
// values in index order: the candidates a top-k sampler draws the next token
// from, selected on the device.
//
// realizar 0.8.5 src/cuda/executor/cached.rs, dispatch_lm_head_and_download:
// the logits go to the host, where the next token is chosen.  With the k
// (index, value) pairs selected here, a sampling step reads back 8 k bytes
// instead of 4 bytes per vocabulary entry.
//
// The order: a ranks above b when a.v > b.v, or a.v == b.v and a.i < b.i, with
// -0 and +0 equal.  Each value becomes a 32-bit key that orders the same way
// (zero made +0, then the sign bit flipped for non-negative values and every
// bit flipped for negative ones), so the selection is over (key desc, index
// asc): a strict total order on distinct indices, hence one answer.
//
// Selection without sorting.  A workgroup holds a list of keys in registers,
// thread t owning list positions t E .. t E + E - 1, some of them marked as
// taking part.  It finds the k-th largest key T among those by radix select
// over a key interval [lo, hi] that holds it, starting from the smallest and
// largest key present: each round cuts the interval into at most 2048 equal
// bins of a power-of-two width, counts the keys in each (an LDS histogram)
// and keeps the bin that holds the k-th largest.  A bin of width one is T
// itself; a bin whose keys are exactly those still wanted ends the search
// early.  The width shrinks by 2^11 a round, so three rounds cover 32 bits,
// and bins spread over the keys actually present, which keeps few lanes of a
// wave on one LDS address.  Then one prefix sum over the threads writes, in
// list order, every key above the interval and the first (still wanted) keys
// inside it: exactly k entries, ties taken in list order, which is index
// order.
//
// Two kernels.  (1) One workgroup per slice of kTopkSlice values keeps the
// slice's k selected entries (a last slice of r < k values keeps its r and
// fills the other slots with key 0 and index kTopkNone, which take no part
// later).  The slices' entries, concatenated, are in index order and hold the
// whole array's top k.  (2) One workgroup selects k of them the same way,
// ranks the k against each other, and writes indices and values largest
// first.  Both are short chains of barrier-separated phases whose cost is
// instruction issue rather than memory: the loops over a thread's entries are
// fully unrolled (no branches, no waits between LDS reads), scans use DPP
// lane moves, and the merge's shape (threads, entries a thread) is chosen
// from the candidate count so that no wave walks entries that cannot exist.
#include "rz_device.h"
#include "rz_launch.h"

namespace rz {

constexpr int kTopkBins = 2048;                 // 11-bit digits
constexpr unsigned kTopkNone = 0x7fffffffu;     // index of a padding entry (key 0)
constexpr int kSliceThreads = 256, kSliceE = kTopkSlice / kSliceThreads;
static_assert(kSliceThreads * kSliceE == kTopkSlice, "");

__device__ __forceinline__ unsigned topk_key(float v) {
  unsigned u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;   // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// DPP lane moves (gfx9 encodings): row_shr:n is 0x110 + n, row_bcast:15 is
// 0x142, row_bcast:31 is 0x143.  A lane whose source lies outside its row, or
// whose row is masked off, gets `id`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ unsigned topk_dpp(unsigned id, unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive scan over the wave's 64 lanes with an associative op whose
// identity is id: within rows of 16 by shifts of 1, 2, 4, 8, then the row
// totals carried across rows.
template <typename Op>
__device__ __forceinline__ unsigned topk_wave_scan(unsigned x, unsigned id, Op op) {
  x = op(x, topk_dpp<0x111, 0xf>(id, x));
  x = op(x, topk_dpp<0x112, 0xf>(id, x));
  x = op(x, topk_dpp<0x114, 0xf>(id, x));
  x = op(x, topk_dpp<0x118, 0xf>(id, x));
  x = op(x, topk_dpp<0x142, 0xa>(id, x));
  x = op(x, topk_dpp<0x143, 0xc>(id, x));
  return x;
}

struct TopkAdd {
  __device__ unsigned operator()(unsigned a, unsigned b) const { return a + b; }
};
struct TopkMin {
  __device__ unsigned operator()(unsigned a, unsigned b) const { return min(a, b); }
};
struct TopkMax {
  __device__ unsigned operator()(unsigned a, unsigned b) const { return max(a, b); }
};

template <int THREADS>
struct TopkShared {
  unsigned hist[3][kTopkBins];   // one per radix round, cleared up front
  unsigned wave_lo[THREADS / kWave], wave_hi[THREADS / kWave], wave_sum[THREADS / kWave];
  unsigned bin, above, in_bin;
};

// Smallest and largest of the taking-part keys (at least one) over the
// workgroup; also clears the histograms.  Ends past one barrier.
template <int THREADS, int E>
__device__ __forceinline__ void topk_range(const unsigned (&key)[E], const bool (&on)[E], int ne,
                                           TopkShared<THREADS>& sh, unsigned& lo, unsigned& hi) {
  for (int b = (int)threadIdx.x; b < 3 * kTopkBins; b += THREADS) (&sh.hist[0][0])[b] = 0;
  unsigned a = 0xffffffffu, z = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e >= ne) continue;
    if (on[e]) {
      a = min(a, key[e]);
      z = max(z, key[e]);
    }
  }
  a = (unsigned)__builtin_amdgcn_readlane((int)topk_wave_scan(a, 0xffffffffu, TopkMin()), kWave - 1);
  z = (unsigned)__builtin_amdgcn_readlane((int)topk_wave_scan(z, 0u, TopkMax()), kWave - 1);
  const int wave = (int)threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.wave_lo[wave] = a;
    sh.wave_hi[wave] = z;
  }
  __syncthreads();
  lo = 0xffffffffu;
  hi = 0u;
#pragma unroll
  for (int w = 0; w < THREADS / kWave; ++w) {
    lo = min(lo, sh.wave_lo[w]);
    hi = max(hi, sh.wave_hi[w]);
  }
}

// Histogram word of bin b.  Bins go in blocks of 32 (block b / 32 is summed
// by one lane in topk_pick); a block's eight groups of four bins are stored in
// an order that depends on the block, so that the lanes' 16-byte reads of one
// group index fall in different LDS banks while each lane still receives its
// groups in bin order.
__device__ __forceinline__ unsigned topk_bin_word(unsigned b) {
  const unsigned rot = (b >> 6) & 7u;   // ((b / 32) >> 1) & 7
  return (b & ~31u) | ((((b >> 2) & 7u) ^ rot) << 2) | (b & 3u);
}

// The bin of `hist` (laid out by topk_bin_word) that holds the need-th
// largest key counted, with the count above it and its own count; found by
// the calling wave alone, the same in all its lanes.  1 <= need <= keys
// counted.  First the block of 32 bins (one lane per block, a scan over the
// block totals from the top), then the bin inside it (one lane per bin, a
// second scan).
__device__ __forceinline__ void topk_pick(const unsigned* hist, unsigned need, unsigned& bin,
                                          unsigned& above, unsigned& in_bin) {
  const int lane = (int)threadIdx.x & (kWave - 1);
  const int blk = kWave - 1 - lane;   // lane 0 holds the top block
  const int rot = (blk >> 1) & 7;
  const uint4* q = reinterpret_cast<const uint4*>(hist + 32 * blk);
  unsigned s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint4 g = q[j ^ rot];
    s += g.x + g.y + g.z + g.w;
  }
  const unsigned incl = topk_wave_scan(s, 0u, TopkAdd());
  const unsigned long long hit = __ballot(incl - s < need && need <= incl);
  const int src = __ffsll((unsigned long long)hit) - 1;   // exactly one lane
  const unsigned top_blk = (unsigned)(kWave - 1 - src);
  const unsigned pre = (unsigned)__builtin_amdgcn_readlane((int)(incl - s), src);
  // lane l < 32 takes bin 32 top_blk + 31 - l: the block's bins from the top
  const unsigned my_bin = 32u * top_blk + 31u - (unsigned)(lane & 31);
  const unsigned c = lane < 32 ? hist[topk_bin_word(my_bin)] : 0u;
  const unsigned run = pre + topk_wave_scan(c, 0u, TopkAdd());
  const unsigned long long hit2 = __ballot(lane < 32 && run >= need);
  const int f = __ffsll((unsigned long long)hit2) - 1;   // a lane below 32
  bin = (unsigned)__builtin_amdgcn_readlane((int)my_bin, f);
  in_bin = (unsigned)__builtin_amdgcn_readlane((int)c, f);
  above = (unsigned)__builtin_amdgcn_readlane((int)(run - c), f);
}

// Radix select over the taking-part keys: on return every one of them in
// [lo, hi] is a candidate for the last `need` places, `need` of them complete
// the selection, and the k - need above hi are selected.  1 <= k <= number of
// taking-part keys.  EVERY_WAVE: each wave finds the bin itself (one barrier
// a round); otherwise wave 0 finds it and passes it on through LDS.
template <int THREADS, int E, bool EVERY_WAVE>
__device__ __forceinline__ void topk_select(const unsigned (&key)[E], const bool (&on)[E], int ne,
                                            int k, TopkShared<THREADS>& sh, unsigned& lo,
                                            unsigned& hi, int& need) {
  topk_range<THREADS, E>(key, on, ne, sh, lo, hi);
  need = k;
  for (int r = 0; r < 3; ++r) {
    const unsigned span = hi - lo;
    const int len = span ? 32 - __clz((int)span) : 0;
    const int shift = len > 11 ? len - 11 : 0;   // (span >> shift) < kTopkBins
    unsigned* hist = sh.hist[r];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e >= ne) continue;
      if (on[e] && key[e] >= lo && key[e] <= hi)
        atomicAdd(&hist[topk_bin_word((key[e] - lo) >> shift)], 1u);
    }
    __syncthreads();
    unsigned bin, above, in_bin;
    if (EVERY_WAVE) {
      topk_pick(hist, (unsigned)need, bin, above, in_bin);
    } else {
      if (threadIdx.x < kWave) {
        topk_pick(hist, (unsigned)need, bin, above, in_bin);
        if (threadIdx.x == 0) {
          sh.bin = bin;
          sh.above = above;
          sh.in_bin = in_bin;
        }
      }
      __syncthreads();
      bin = sh.bin;
      above = sh.above;
      in_bin = sh.in_bin;
      // sh.bin is written again after the next round's barrier, which every
      // thread reaches after reading it here
    }
    const unsigned nlo = lo + (bin << shift);
    const unsigned width_m1 = (1u << shift) - 1u;
    hi = hi - nlo < width_m1 ? hi : nlo + width_m1;
    lo = nlo;
    need -= (int)above;
    // every key left in the bin is selected, or the bin is one key: no
    // further digit to fix
    if ((int)in_bin == need || shift == 0) break;
  }
}

// Calls put(pos, key, index) for the k selected entries, pos = their order
// in the list (0 .. k-1).
template <int THREADS, int E, typename Put>
__device__ __forceinline__ void topk_compact(const unsigned (&key)[E], const unsigned (&idx)[E],
                                             const bool (&on)[E], int ne, unsigned lo,
                                             unsigned hi, int need, TopkShared<THREADS>& sh,
                                             Put put) {
  unsigned cg = 0, ce = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e >= ne) continue;
    cg += on[e] && key[e] > hi;
    ce += on[e] && key[e] >= lo && key[e] <= hi;
  }
  // counts <= kTopkMerge < 2^16: two fields in one scan
  const unsigned v = cg | (ce << 16);
  const unsigned incl = topk_wave_scan(v, 0u, TopkAdd());
  const int wave = (int)threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == kWave - 1) sh.wave_sum[wave] = incl;
  __syncthreads();
  unsigned pre = incl - v;
#pragma unroll
  for (int w = 0; w < THREADS / kWave; ++w) pre += w < wave ? sh.wave_sum[w] : 0u;
  unsigned g_before = pre & 0xffffu, e_before = pre >> 16;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e >= ne) continue;
    const bool gt = on[e] && key[e] > hi, eq = on[e] && key[e] >= lo && key[e] <= hi;
    if (gt || (eq && e_before < (unsigned)need))
      put(g_before + min(e_before, (unsigned)need), key[e], idx[e]);
    g_before += gt;
    e_before += eq;
  }
}

__global__ __launch_bounds__(kSliceThreads) void topk_slice_kernel(const float* __restrict__ v,
                                                                   int n, int k,
                                                                   unsigned* __restrict__ cand_key,
                                                                   int* __restrict__ cand_idx) {
  __shared__ __align__(16) TopkShared<kSliceThreads> sh;
  const long base = (long)blockIdx.x * kTopkSlice;
  const long first = base + (long)threadIdx.x * kSliceE;
  unsigned key[kSliceE], idx[kSliceE];
  bool on[kSliceE];
  if (base + kTopkSlice <= n) {   // a whole slice: 16-byte loads
    static_assert(kSliceE % 4 == 0, "");
#pragma unroll
    for (int e = 0; e < kSliceE; e += 4) {
      const u32x4_a4 q = *reinterpret_cast<const u32x4_a4*>(v + first + e);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        key[e + c] = topk_key(__uint_as_float(q[c]));
        idx[e + c] = (unsigned)(first + e + c);
        on[e + c] = true;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kSliceE; ++e) {
      const long i = first + e;
      on[e] = i < n;
      key[e] = on[e] ? topk_key(v[i]) : 0u;
      idx[e] = on[e] ? (unsigned)i : kTopkNone;
    }
  }
  const int real = (int)min((long)kTopkSlice, (long)n - base);
  const int ks = min(k, real);
  unsigned lo, hi;
  int need;
  topk_select<kSliceThreads, kSliceE, true>(key, on, kSliceE, ks, sh, lo, hi, need);
  unsigned* ok = cand_key + base / kTopkSlice * k;
  int* oi = cand_idx + base / kTopkSlice * k;
  topk_compact<kSliceThreads, kSliceE>(key, idx, on, kSliceE, lo, hi, need, sh,
                                       [&](unsigned pos, unsigned kk, unsigned ii) {
                                         if (pos < (unsigned)ks) {
                                           ok[pos] = kk;
                                           oi[pos] = (int)ii;
                                         }
                                       });
  for (int t = ks + (int)threadIdx.x; t < k; t += kSliceThreads) {
    ok[t] = 0u;
    oi[t] = (int)kTopkNone;
  }
}

// NE candidates a thread (THREADS NE >= m): thread t holds candidates
// t NE .. t NE + NE - 1, read 16 bytes at a time.  The launcher picks the
// shape by m, so that no thread walks slots that cannot hold a candidate.
template <int THREADS, int NE>
__global__ __launch_bounds__(THREADS) void topk_merge_kernel(
    const float* __restrict__ v, int n, const unsigned* __restrict__ cand_key,
    const int* __restrict__ cand_idx, int m, int k, int* __restrict__ out_i,
    float* __restrict__ out_v) {
  constexpr int E = NE, ne = NE;
  static_assert(E % 4 == 0, "");
  __shared__ __align__(16) TopkShared<THREADS> sh;
  __shared__ __align__(16) unsigned sel_key[kTopkMaxK];
  __shared__ __align__(16) unsigned sel_idx[kTopkMaxK];
  const int first = (int)threadIdx.x * NE;
  unsigned key[E], idx[E];
  bool on[E];
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    if (first + e + 4 <= m) {
      const u32x4_a4 qk = *reinterpret_cast<const u32x4_a4*>(cand_key + first + e);
      const u32x4_a4 qi = *reinterpret_cast<const u32x4_a4*>(cand_idx + first + e);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        key[e + c] = qk[c];
        idx[e + c] = qi[c];
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool in = first + e + c < m;
        key[e + c] = in ? cand_key[first + e + c] : 0u;
        idx[e + c] = in ? (unsigned)cand_idx[first + e + c] : kTopkNone;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) on[e] = idx[e] != kTopkNone;
  unsigned lo, hi;
  int need;
  topk_select<THREADS, E, false>(key, on, ne, k, sh, lo, hi, need);
  topk_compact<THREADS, E>(key, idx, on, ne, lo, hi, need, sh,
                           [&](unsigned pos, unsigned kk, unsigned ii) {
                             if (pos < (unsigned)k) {
                               sel_key[pos] = kk;
                               sel_idx[pos] = ii;
                             }
                           });
  __syncthreads();
  // Each selected entry's place is the number of selected entries ranked
  // above it: THREADS / kTopkMaxK threads per entry, each comparing it with
  // every such share of the others (four a read), then summed over the share
  // group's adjacent lanes.
  constexpr int PARTS = THREADS / kTopkMaxK;
  static_assert(PARTS >= 1 && PARTS <= 16 && (PARTS & (PARTS - 1)) == 0, "");
  const int t = (int)threadIdx.x / PARTS, part = (int)threadIdx.x % PARTS;
  const unsigned a = t < k ? sel_key[t] : 0u, ai = t < k ? sel_idx[t] : 0u;
  int rank = 0;
  if (t < k) {
#pragma unroll 2
    for (int j = 4 * part; j < k; j += 4 * PARTS) {
      const uint4 bk = *reinterpret_cast<const uint4*>(&sel_key[j]);
      const uint4 bi = *reinterpret_cast<const uint4*>(&sel_idx[j]);
      rank += (int)((j + 0 < k) & ((bk.x > a) | ((bk.x == a) & (bi.x < ai))));
      rank += (int)((j + 1 < k) & ((bk.y > a) | ((bk.y == a) & (bi.y < ai))));
      rank += (int)((j + 2 < k) & ((bk.z > a) | ((bk.z == a) & (bi.z < ai))));
      rank += (int)((j + 3 < k) & ((bk.w > a) | ((bk.w == a) & (bi.w < ai))));
    }
  }
#pragma unroll
  for (int d = 1; d < PARTS; d <<= 1) rank += __shfl_xor(rank, d, kWave);
  if (t < k && part == 0) {
    if (out_i) out_i[rank] = (int)ai;
    if (out_v && ai < (unsigned)n) out_v[rank] = v[ai];
  }
}

long topk_slices(int n) { return ((long)n + kTopkSlice - 1) / kTopkSlice; }

hipError_t launch_topk_f32(const float* v, int n, int k, int* out_i, float* out_v,
                           unsigned* cand_key, int* cand_idx, hipStream_t st) {
  const long g = topk_slices(n);
  const long m = g * k;
  if (n < 1 || k < 1 || k > kTopkMaxK || k > n || m > kTopkMerge) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_slice_kernel, dim3((unsigned)g), dim3(kSliceThreads), 0, st, v, n, k,
                     cand_key, cand_idx);
  const unsigned* ck = cand_key;
  const int* ci = cand_idx;
  const dim3 grid(1);
#define RZ_TOPK_MERGE(T, NE) \
  hipLaunchKernelGGL((topk_merge_kernel<T, NE>), grid, dim3(T), 0, st, v, n, ck, ci, (int)m, k, out_i, out_v)
  // shapes by measured time per candidate count (fewer waves while the
  // per-wave fixed work dominates, more once the slots do)
  if (m <= 2048)
    RZ_TOPK_MERGE(512, 4);
  else if (m <= 4096)
    RZ_TOPK_MERGE(1024, 4);
  else if (m <= 8192)
    RZ_TOPK_MERGE(1024, 8);
  else
    RZ_TOPK_MERGE(1024, 16);
#undef RZ_TOPK_MERGE
  static_assert(1024 * 16 == kTopkMerge, "");
  return hipGetLastError();
}

}  // namespace rz
