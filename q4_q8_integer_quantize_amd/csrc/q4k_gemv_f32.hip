// q4k_gemv_f32.hip -- y = W Q8_1(x) for an fp32 activation x, quantize and GEMV
// in one launch.
//
// realizar 0.8.5 src/cuda/executor/cached.rs, transformer_layer_gpu_true_dp4a,
// steps 2-3: the normed activation is quantized to Q8_1 and multiplied by the
// Q4_K weights with integer dot products.  Here every workgroup quantizes the
// (short) activation itself, into LDS, with the same block rule as
// rz_q8_1_quantize, while its first weight tiles are already on their way from
// HBM; a separate quantize launch would cost a whole kernel boundary on every
// GEMV.  The result is bit-identical to rz_q8_1_quantize followed by
// rz_q4k_q8_gemv, and workgroup 0 can also write the Q8_1 blocks out so that
// further projections of the same activation (K, V after Q) reuse them.
//
// When n is a multiple of 4 (XV) every thread's four values of a pass come in
// one 16-byte load; otherwise as four dword loads, so a quad that straddles n
// reads zeros past it.  The activation loads go out first and as few as
// possible: at kernel start they compete with the first weight tiles.
//
// Order inside a workgroup: (1) the lane's share of x is requested, (2) the
// first weight tiles are requested, (3) x is quantized into LDS as soon as it
// arrives (vector loads retire in order, so this wait does not include the
// weight tiles), (4) an LDS-only barrier, (5) the GEMV pipeline of
// q4k_q8_gemv_kernel.
//
// RES adds a residual in the store, y = W Q8_1(x) + r (cached.rs steps 5-7:
// the attention output quantized for the O projection, whose result is added
// to the hidden state), with r's values requested right after each weight tile
// as in q4k_q8_gemv_kernel; r may be y itself.
#include "q4k_gemv.h"
#include "rz_launch.h"

namespace rz {

struct Q4KF32Args {
  const uint8_t* w;
  const float* x;     // fp32 [n] (zero-padded to in_dim on the fly)
  uint8_t* xq_out;    // optional Q8_1 [in_dim/32] blocks
  float* y;
  int n;
  int out_dim;
  int nsb;            // super-blocks per row (in_dim / 256)
  const float* r;     // RES: residual [out_dim] (may be y), else unused
};

// Activation slots from the workgroup's LDS copy of the Q8_1 blocks, which
// holds all S * TPR slots (zero blocks past the row), so no slot is tested.
template <int TPR, int S>
__device__ __forceinline__ void load_x_slots_lds(XSlots<S, 1>& xs, const uint8_t* xq, int nsb,
                                                 const LaneRole& ro) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int sb = s * TPR + ro.tslot;
    (void)nsb;   // the LDS copy holds all S * TPR slots, zero blocks past nsb
    {
      const uint8_t* xb = xq + sb * 8 * kQ8Bytes;
      const uint2* plo = (const uint2*)(xb + (2 * ro.c) * kQ8Bytes + 8 + 16 * ro.h);
      const uint2* phi = (const uint2*)(xb + (2 * ro.c + 1) * kQ8Bytes + 8 + 16 * ro.h);
      const uint2 a0 = plo[0], a1 = plo[1], b0 = phi[0], b1 = phi[1];
      xs.lo[0][s][0] = (int)a0.x; xs.lo[0][s][1] = (int)a0.y;
      xs.lo[0][s][2] = (int)a1.x; xs.lo[0][s][3] = (int)a1.y;
      xs.hi[0][s][0] = (int)b0.x; xs.hi[0][s][1] = (int)b0.y;
      xs.hi[0][s][2] = (int)b1.x; xs.hi[0][s][3] = (int)b1.y;
      const float* own = (const float*)(xb + ro.i * kQ8Bytes);
      xs.dx[0][s] = own[0];
      xs.sx[0][s] = own[1];
    }
  }
}

// Q8_1 blocks per workgroup pass: 8 lanes per block, WPB waves.
template <int WPB>
constexpr int blocks_per_pass() { return 8 * WPB; }

template <int TPR, int S, int R, int G, int P, bool XV, int WPB = 4, bool RES = false>
__global__ __launch_bounds__(64 * WPB) void q4k_gemv_f32_kernel(Q4KF32Args a) {
  constexpr int kBlocksPerPass = blocks_per_pass<WPB>();
  constexpr int RW = 8 / TPR;
  constexpr uint32_t kRowsPerGroup = (uint32_t)RW * R;
  // the longest activation this instantiation serves: S slots of TPR teams
  constexpr int kPasses = (S * TPR * 8 + kBlocksPerPass - 1) / kBlocksPerPass;
  extern __shared__ __attribute__((aligned(16))) uint8_t xq_lds[];

  const int nblk = a.nsb * 8;
  const int qi = threadIdx.x & 7;   // lane within its quantize group
  const int qb = threadIdx.x >> 3;  // block within a pass

  // (1) this thread's share of x: 4 values of block p*32 + qb per pass
  const uint32_t xbytes = (uint32_t)a.n * 4u;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, (int)xbytes, kBufferWord3);
  float xv[kPasses][4];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int b = p * kBlocksPerPass + qb;
    if constexpr (XV) {
      const uint32_t e = (uint32_t)(b * kQK8 + 4 * qi);
      const uint32_t off = (b < nblk && e < (uint32_t)a.n) ? e * 4u : xbytes;
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
      // copy the elements out before reinterpreting them
      const uint32_t v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
      xv[p][0] = __builtin_bit_cast(float, v0);
      xv[p][1] = __builtin_bit_cast(float, v1);
      xv[p][2] = __builtin_bit_cast(float, v2);
      xv[p][3] = __builtin_bit_cast(float, v3);
    } else {
      load_block_quad(xv[p], xr, 0u, b * kQK8 + 4 * qi, a.n, b < nblk, xbytes);
    }
  }

  // (2) the first weight tiles
  const uint32_t nwaves = gridDim.x * (uint32_t)WPB;
  const uint32_t wid =
      __builtin_amdgcn_readfirstlane(blockIdx.x * (uint32_t)WPB + (threadIdx.x >> 6));
  const LaneRole ro = make_role<TPR>();
  const uint32_t row_bytes = (uint32_t)a.nsb * kQ4KBytes;
  const WSrc src = make_wsrc(a.w, row_bytes, (uint32_t)a.out_dim * row_bytes);
  const LaneOffsets<TPR, S> off = lane_offsets<TPR, S>(src, 0, ro);
  Q4KGemvArgs ga;
  ga.r = a.r;
  ga.w = a.w;
  ga.xq = nullptr;
  ga.y = a.y;
  ga.out_dim = a.out_dim;
  ga.nsb_row = a.nsb;
  ga.sb0 = 0;
  ga.nsb = a.nsb;
  ga.n_tokens = 1;
  WTile<S, R> t[G];
  float rv[G][R][1];
  __amdgpu_buffer_rsrc_t rr;
  if constexpr (RES)
    rr = __builtin_amdgcn_make_buffer_rsrc((void*)a.r, (short)0, (int)((uint32_t)a.out_dim * 4u),
                                           kBufferWord3);
#pragma unroll
  for (int k = 0; k < P && k < G; ++k) {
    load_w_tile<TPR, S, R>(t[k], src, off, (wid + k * nwaves) * kRowsPerGroup);
    if constexpr (RES)
      load_residual<TPR, R, 1>(rv[k], rr, ga, (long)(wid + k * nwaves) * kRowsPerGroup, ro);
  }
  __builtin_amdgcn_sched_barrier(0);

  // (3) quantize into LDS (and, in workgroup 0, to global memory); the LDS copy
  // covers all S * TPR slots, and blocks past nblk quantize zeros into zero blocks
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int b = p * kBlocksPerPass + qb;
    if (b < S * TPR * 8) {   // whole 8-lane groups take the same branch
      float d, s;
      const uint32_t packed = q8_1_block_group8(xv[p], d, s);
      uint8_t* blk = xq_lds + b * kQ8Bytes;
      *(uint32_t*)(blk + 8 + 4 * qi) = packed;
      if (qi == 0) {
        ((float*)blk)[0] = d;
        ((float*)blk)[1] = s;
      }
      if (a.xq_out && blockIdx.x == 0 && b < nblk) {
        uint8_t* g = a.xq_out + (size_t)b * kQ8Bytes;
        *(uint32_t*)(g + 8 + 4 * qi) = packed;
        if (qi == 0) {
          ((float*)g)[0] = d;
          ((float*)g)[1] = s;
        }
      }
    }
  }
  // (4) LDS-only release/acquire around the barrier: the weight loads stay in
  // flight (a full fence would wait for them)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  // (5) GEMV over the register-resident slots
  XSlots<S, 1> xs;
  load_x_slots_lds<TPR, S>(xs, xq_lds, a.nsb, ro);
#pragma unroll
  for (int k = 0; k < G; ++k) {
    if (k + P < G) {
      load_w_tile<TPR, S, R>(t[k + P], src, off, (wid + (k + P) * nwaves) * kRowsPerGroup);
      if constexpr (RES)
        load_residual<TPR, R, 1>(rv[k + P], rr, ga, (long)(wid + (k + P) * nwaves) * kRowsPerGroup,
                                 ro);
    }
    __builtin_amdgcn_sched_barrier(0);
    float acc[R][1];
    q4k_tile_dot<TPR, S, R, 1>(acc, t[k], xs, ro);
    if constexpr (RES)
      store_rows_residual<TPR, R, 1>(ga, acc, rv[k], (long)(wid + k * nwaves) * kRowsPerGroup, ro);
    else
      store_rows<TPR, R, 1, false>(ga, acc, (long)(wid + k * nwaves) * kRowsPerGroup, ro);
  }
}

constexpr int kF32TilesInFlight = 2;
// About one wave per SIMD: 256 CUs x 4 SIMDs.  Each workgroup quantizes the
// whole activation, so the grid stays near one 4-wave workgroup per CU.
constexpr long kF32TargetWaves = 1024;

template <int TPR, int S, int G, bool XV, int WPB = 4>
static hipError_t launch_f32_g(const Q4KF32Args& a, long groups, hipStream_t st) {
  constexpr int R = S <= 2 ? 2 : 1;
  constexpr int P = G > kF32TilesInFlight ? kF32TilesInFlight : (G > 1 ? G - 1 : 1);
  const long waves = (groups + G - 1) / G;
  const unsigned grid = (unsigned)((waves + WPB - 1) / WPB);
  const size_t lds = (size_t)S * TPR * 8 * kQ8Bytes;
  if (a.r)
    hipLaunchKernelGGL((q4k_gemv_f32_kernel<TPR, S, R, G, P, XV, WPB, true>), dim3(grid),
                       dim3(64 * WPB), lds, st, a);
  else
    hipLaunchKernelGGL((q4k_gemv_f32_kernel<TPR, S, R, G, P, XV, WPB>), dim3(grid), dim3(64 * WPB),
                       lds, st, a);
  return hipGetLastError();
}

// G (row groups a wave) is the smallest count that keeps the grid within the
// target, not rounded to a power of two: 14336 rows are 7168 groups, so G = 7
// gives 256 workgroups, one for every CU, where G = 8 left 32 CUs without work
// (measured on the 4096 -> 14336 step: 7.40 against 7.57 us, kernel trace
// 7.59 against 7.97 us).
template <int TPR, int S, bool XV>
static hipError_t run_f32_x(const Q4KF32Args& a, hipStream_t st) {
  constexpr int R = S <= 2 ? 2 : 1;
  constexpr int RW = 8 / TPR;
  const long rows_per_group = (long)RW * R;
  const long groups = (a.out_dim + rows_per_group - 1) / rows_per_group;
  const long per_wave = (groups + kF32TargetWaves - 1) / kF32TargetWaves;
  switch (per_wave) {
    case 1: return launch_f32_g<TPR, S, 1, XV>(a, groups, st);
    case 2: return launch_f32_g<TPR, S, 2, XV>(a, groups, st);
    case 3: return launch_f32_g<TPR, S, 3, XV>(a, groups, st);
    case 4: return launch_f32_g<TPR, S, 4, XV>(a, groups, st);
    case 5: return launch_f32_g<TPR, S, 5, XV>(a, groups, st);
    case 6: return launch_f32_g<TPR, S, 6, XV>(a, groups, st);
    case 7: return launch_f32_g<TPR, S, 7, XV>(a, groups, st);
    default: return launch_f32_g<TPR, S, 8, XV>(a, groups, st);
  }
}

template <int TPR, int S>
static hipError_t run_f32(const Q4KF32Args& a, hipStream_t st) {
  return (a.n & 3) == 0 ? run_f32_x<TPR, S, true>(a, st) : run_f32_x<TPR, S, false>(a, st);
}

hipError_t launch_q4k_q8_gemv_f32(const uint8_t* w, const float* x, int n, uint8_t* xq_out,
                                  float* y, int out_dim, int in_dim, hipStream_t stream,
                                  const float* r) {
  Q4KF32Args a;
  a.r = r;
  a.w = w;
  a.x = x;
  a.xq_out = xq_out;
  a.y = y;
  a.n = n;
  a.out_dim = out_dim;
  a.nsb = in_dim / kQKK;
  const int nsb = a.nsb;
  if (nsb == 1) return run_f32<1, 1>(a, stream);
  if (nsb == 2) return run_f32<2, 1>(a, stream);
  if (nsb <= 4) return run_f32<4, 1>(a, stream);
  switch ((nsb + 7) / 8) {
    case 1: return run_f32<8, 1>(a, stream);
    case 2: return run_f32<8, 2>(a, stream);
    case 3: return run_f32<8, 3>(a, stream);
    case 4: return run_f32<8, 4>(a, stream);
    case 5: return run_f32<8, 5>(a, stream);
    case 6: return run_f32<8, 6>(a, stream);
    case 7: return run_f32<8, 7>(a, stream);
    case 8: return run_f32<8, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rz
