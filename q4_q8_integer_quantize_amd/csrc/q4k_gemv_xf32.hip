// q4k_gemv_xf32.hip -- Q4_K weights times an fp32 activation, no Q8_1: the
// GEMV and the SwiGLU FFN of the non-quantized activation path.
//
// realizar 0.8.5 src/cuda/executor/cached.rs, transformer_layer_gpu_cached:
// steps 2 and 4 project the fp32 normed activation (q4k_gemv_cached_async,
// tiled_q4k_gemv_cached_async) and step 7 runs the FFN on it
// (fused_ffn_swiglu_gpu); realizar 0.8.4 src/gpu/adapters/using.rs,
// ffn_swiglu_gpu: gate and up GEMVs, the fused SwiGLU, then the down GEMV of
// its fp32 output.
//
// Per 32-value sub-block j of a super-block a lane evaluates, in fp32,
//   d * (sc_j * sum_l q_l x_l) - dmin * (m_j * sum_l x_l)
// (the nibbles enter the fmas exactly, as fp16 denormals q * 2^-24).  Lane roles are
// those of the Q8_1 kernel (q4k_gemv.h): lane i of a team reads qs bytes
// 16i..16i+15, i.e. positions 16h..16h+15 of sub-blocks 2c (low nibbles) and
// 2c+1 (high nibbles), and after adding its partner's half owns sub-block
// j = i.  Its 32 activation values per slot stay in registers.  A row longer
// than the register window (TPR * S super-blocks) is walked in column chunks
// inside the kernel, each row's sum carried in registers from chunk to chunk,
// so one launch covers any in_dim.
//
// SWI: the row groups alternate gate and up rows of the same rows, and the
// epilogue stores h = silu(g) * u = g / (1 + exp(-g)) * u.
#include <utility>

#include "q4k_gemv.h"
#include "rz_launch.h"

namespace rz {

struct XF32Args {
  const uint8_t* w;     // W, or W_gate (SWI)
  const uint8_t* w2;    // W_up (SWI)
  const float* x;       // fp32 [n]; values n .. in_dim-1 read as 0
  float* y;             // y [out_dim], or h [out_dim] (SWI)
  float* gu;            // SWI only, optional: [2][out_dim], g then u
  int n;
  int out_dim;
  int nsb;              // super-blocks per row
};

// The lane's activation values of S slots: lo = sub-block 2c, hi = 2c+1, both
// at positions 16h .. 16h+15; sj = sum of x over the lane's own sub-block.
template <int S>
struct XF32Slots {
  float lo[S][16];
  float hi[S][16];
  float sj[S];
};

// Request slot s's values: super-block sb0 + s*TPR + tslot of the row, for
// the nch super-blocks of this chunk.  XV (n % 4 == 0): 16-byte loads, each
// wholly below n or wholly past it; otherwise dword loads.  Values past n and
// slots past the chunk take the offset xbytes, which reads 0.
template <int TPR, int S, bool XV>
__device__ __forceinline__ void request_x(XF32Slots<S>& xs, __amdgpu_buffer_rsrc_t xr,
                                          uint32_t xbytes, int n, int sb0, int nch,
                                          const LaneRole& ro) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int k = s * TPR + ro.tslot;
    const bool on = k < nch;
    const int base = (sb0 + k) * kQKK + 64 * ro.c + 16 * ro.h;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float* dst = half ? xs.hi[s] : xs.lo[s];
      const int b0 = base + 32 * half;
      if constexpr (XV) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = b0 + 4 * q;
          const uint32_t off = (on && e < n) ? (uint32_t)e * 4u : xbytes;
          const u32x4 v =
              __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
          const uint32_t v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
          dst[4 * q + 0] = __builtin_bit_cast(float, v0);
          dst[4 * q + 1] = __builtin_bit_cast(float, v1);
          dst[4 * q + 2] = __builtin_bit_cast(float, v2);
          dst[4 * q + 3] = __builtin_bit_cast(float, v3);
        }
      } else {
#pragma unroll
        for (int l = 0; l < 16; ++l) {
          const int e = b0 + l;
          const uint32_t off = (on && e < n) ? (uint32_t)e * 4u : xbytes;
          dst[l] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0));
        }
      }
    }
  }
}

__device__ __forceinline__ float xor1_f(float v) { return dpp_f<0xB1>(v); }

// Sum of 16 values as a fixed tree.
__device__ __forceinline__ float sum16(const float (&v)[16]) {
  float a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = v[2 * k] + v[2 * k + 1];
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = a[2 * k] + a[2 * k + 1];
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// sum of x over the sub-block each lane owns (its half plus its partner's);
// then the high-nibble partners are scaled by 2^-4 (exact away from
// underflow), because tile_dot_xf32 takes the high nibbles in place, as
// 16 q * 2^-24.
template <int S>
__device__ __forceinline__ void finish_x(XF32Slots<S>& xs, const LaneRole& ro) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const float sl = sum16(xs.lo[s]), sh = sum16(xs.hi[s]);
    const float keep = ro.h ? sh : sl;
    const float send = ro.h ? sl : sh;
    xs.sj[s] = keep + xor1_f(send);
#pragma unroll
    for (int l = 0; l < 16; ++l) xs.hi[s][l] *= 0x1p-4f;
  }
}

// One tile: part[r] = the row's sum over this chunk, valid in the row's last lane.
template <int TPR, int S, int R>
__device__ __forceinline__ void tile_dot_xf32(float (&part)[R], const WTile<S, R>& wt,
                                              const XF32Slots<S>& xs, const LaneRole& ro) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float a = 0.0f;
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
      // two partial sums per half (even and odd bytes).  The nibbles enter as
      // fp16 denormals, two to a dword, and v_fma_mix_f32 converts them inside
      // the fma (one instruction a weight instead of a byte conversion and an
      // fma): a low nibble masked in place is exactly q * 2^-24, a high nibble
      // masked in place 16 q * 2^-24 against its activation scaled by 2^-4
      // (finish_x), so every product is exactly q * x * 2^-24.  Each partial
      // sum takes the same products in the same order as with fp32 weights,
      // so it is exactly 2^-24 times that sum, and the scale back by 2^24
      // gives the same bits.
      float pl[2] = {0.0f, 0.0f}, ph[2] = {0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = wt.qs[r][s][k];
        const uint32_t w8 = w >> 8;
        const uint32_t l02 = opaque_and(w, 0x000F000Fu);    // low nibbles of bytes 0, 2
        const uint32_t h02 = opaque_and(w, 0x00F000F0u);    // high nibbles of bytes 0, 2, x16
        const uint32_t l13 = opaque_and(w8, 0x000F000Fu);   // low nibbles of bytes 1, 3
        const uint32_t h13 = opaque_and(w8, 0x00F000F0u);   // high nibbles of bytes 1, 3, x16
        pl[0] = fmaf(f16_lo(l02), xs.lo[s][4 * k + 0], pl[0]);
        ph[0] = fmaf(f16_lo(h02), xs.hi[s][4 * k + 0], ph[0]);
        pl[1] = fmaf(f16_lo(l13), xs.lo[s][4 * k + 1], pl[1]);
        ph[1] = fmaf(f16_lo(h13), xs.hi[s][4 * k + 1], ph[1]);
        pl[0] = fmaf(f16_hi(l02), xs.lo[s][4 * k + 2], pl[0]);
        ph[0] = fmaf(f16_hi(h02), xs.hi[s][4 * k + 2], ph[0]);
        pl[1] = fmaf(f16_hi(l13), xs.lo[s][4 * k + 3], pl[1]);
        ph[1] = fmaf(f16_hi(h13), xs.hi[s][4 * k + 3], ph[1]);
      }
      const float sl = (pl[0] + pl[1]) * 0x1p24f;
      const float sh = (ph[0] + ph[1]) * 0x1p24f;
      const float keep = ro.h ? sh : sl;
      const float send = ro.h ? sl : sh;
      const float qx = keep + xor1_f(send);
      a = fmaf((float)d, (float)sc * qx, a);
      a = fmaf((float)dmin, -((float)m * xs.sj[s]), a);
    }
    part[r] = group_sum_dpp<8 * TPR>(a);
  }
}

template <int TPR, int S, int R, int G, int P, bool XV, bool SWI>
__global__ __launch_bounds__(256) void q4k_xf32_kernel(XF32Args a) {
  constexpr int RW = 8 / TPR;
  constexpr uint32_t kRowsPerGroup = (uint32_t)RW * R;
  constexpr int CH = TPR * S;                       // super-blocks per column chunk
  static_assert(!SWI || G % 2 == 0, "gate and up groups come in pairs");
  const uint32_t nwaves = gridDim.x * 4u;
  const uint32_t wid = __builtin_amdgcn_readfirstlane(blockIdx.x * 4u + (threadIdx.x >> 6));
  const LaneRole ro = make_role<TPR>();
  const uint32_t row_bytes = (uint32_t)a.nsb * kQ4KBytes;
  const uint32_t wbytes = (uint32_t)a.out_dim * row_bytes;
  const WSrc src = make_wsrc(a.w, row_bytes, wbytes);
  const WSrc src2 = make_wsrc(SWI ? a.w2 : a.w, row_bytes, wbytes);
  const uint32_t xbytes = (uint32_t)a.n * 4u;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, (int)xbytes, kBufferWord3);
  // first row of step k's group: a strided group of the wave (SWI: gate and
  // up of the same group in steps 2p, 2p+1)
  auto group_row = [&](int k) -> uint32_t {
    const uint32_t gi = SWI ? (uint32_t)(k >> 1) : (uint32_t)k;
    return (wid + gi * nwaves) * kRowsPerGroup;
  };
  auto src_of = [&](int k) -> const WSrc& { return (SWI && (k & 1)) ? src2 : src; };

  float acc[G][R];
#pragma unroll
  for (int k = 0; k < G; ++k)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[k][r] = 0.0f;

  for (int sb0 = 0; sb0 < a.nsb; sb0 += CH) {
    const int nch = a.nsb - sb0 < CH ? a.nsb - sb0 : CH;
    // slots past the chunk read nothing (their offset is past the matrix)
    LaneOffsets<TPR, S> off;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int k = s * TPR + ro.tslot;
      off.hd[s] = k < nch ? (uint32_t)ro.rs * row_bytes + (uint32_t)(sb0 + k) * kQ4KBytes : wbytes;
      off.qs[s] = k < nch ? off.hd[s] + 16u + 16u * (uint32_t)ro.i : wbytes;
    }
    // activation first: vector loads retire in order
    XF32Slots<S> xs;
    request_x<TPR, S, XV>(xs, xr, xbytes, a.n, sb0, nch, ro);
    WTile<S, R> t[G];
#pragma unroll
    for (int k = 0; k < P && k < G; ++k) load_w_tile<TPR, S, R>(t[k], src_of(k), off, group_row(k));
    __builtin_amdgcn_sched_barrier(0);
    finish_x<S>(xs, ro);
#pragma unroll
    for (int k = 0; k < G; ++k) {
      if (k + P < G) load_w_tile<TPR, S, R>(t[k + P], src_of(k + P), off, group_row(k + P));
      __builtin_amdgcn_sched_barrier(0);
      float part[R];
      tile_dot_xf32<TPR, S, R>(part, t[k], xs, ro);
#pragma unroll
      for (int r = 0; r < R; ++r) acc[k][r] += part[r];
    }
  }

  if (!row_leader<TPR>(ro)) return;
  if constexpr (!SWI) {
#pragma unroll
    for (int k = 0; k < G; ++k)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t row = group_row(k) + (uint32_t)(r * RW + ro.rs);
        if (row < (uint32_t)a.out_dim) a.y[row] = acc[k][r];
      }
  } else {
#pragma unroll
    for (int p = 0; p < G / 2; ++p)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t row = group_row(2 * p) + (uint32_t)(r * RW + ro.rs);
        if (row < (uint32_t)a.out_dim) {
          const float g = acc[2 * p][r], u = acc[2 * p + 1][r];
          a.y[row] = g / (1.0f + expf(-g)) * u;
          if (a.gu) {
            a.gu[row] = g;
            a.gu[(size_t)a.out_dim + row] = u;
          }
        }
      }
  }
}

template <int TPR, int S, int R, int G, bool SWI>
static hipError_t launch_xf32_g(const XF32Args& a, long groups, hipStream_t st) {
  constexpr int P = G > 2 ? 2 : (G > 1 ? G - 1 : 1);
  const long steps = SWI ? 2 * groups : groups;
  const long waves = (steps + G - 1) / G;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  if (a.n % 4 == 0)
    hipLaunchKernelGGL((q4k_xf32_kernel<TPR, S, R, G, P, true, SWI>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((q4k_xf32_kernel<TPR, S, R, G, P, false, SWI>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Steps a wave (SWI: even, a gate and an up group per pair), 1..16: the count
// that gives the CUs the smallest even share of steps, ceil(workgroups / 256)
// * 4 waves * G, the larger count on a tie.  Measured in one process, outputs
// bit-identical, against the former rule (the smallest power of two up to 8
// that keeps about 1024 waves):
//   GEMV 4096 -> 14336:    G = 14 (256 workgroups) 8.9-9.5 us; G = 8 9.8-10.0, 7 9.4-9.6, 4 10.4-10.6
//   GEMV 4096 -> 11008:    G = 11 (251)            7.7-7.8 us; G = 8 9.6-9.8, 12 8.0, 6 8.3
//   gate/up 4096 -> 14336: G = 14 (512)          16.0-16.1 us; G = 8 17.5-17.6, 28 17.5-18.0, 6 17.4-17.9
//   gate/up 4096 -> 11008: G = 12 (459)          13.9 us;      G = 8 14.2-14.5, 6 14.3, 14 14.8
static int xf32_steps_per_wave(long steps, bool swi) {
  int best = swi ? 2 : 1;
  long best_share = -1;
  for (int g = best; g <= 16; g += swi ? 2 : 1) {
    const long wgs = ((steps + g - 1) / g + 3) / 4;
    const long share = (wgs + 255) / 256 * 4L * g;
    if (best_share < 0 || share <= best_share) {
      best = g;
      best_share = share;
    }
  }
  return best;
}

template <int TPR, int S, int R, bool SWI, int... Is>
static hipError_t launch_xf32_any(int g, const XF32Args& a, long groups, hipStream_t st,
                                  std::integer_sequence<int, Is...>) {
  // candidate i is G = i + 1, or 2 (i + 1) for SWI
  hipError_t e = hipErrorInvalidValue;
  ((g == (SWI ? 2 : 1) * (Is + 1) ? (e = launch_xf32_g<TPR, S, R, (SWI ? 2 : 1) * (Is + 1), SWI>(a, groups, st), 0)
                                  : 0),
   ...);
  return e;
}

// Rows per group: two for the one-slot window, one for the two-slot window
// (measured at 4096 -> 14336: 9.9 us against 11.0 for two rows, whose extra
// tile registers cost occupancy).
template <int TPR, int S, bool SWI>
static hipError_t run_xf32(const XF32Args& a, hipStream_t st) {
  constexpr int R = S == 1 ? 2 : 1;
  constexpr long rows_per_group = (long)(8 / TPR) * R;
  const long groups = (a.out_dim + rows_per_group - 1) / rows_per_group;
  const int g = xf32_steps_per_wave(SWI ? 2 * groups : groups, SWI);
  return launch_xf32_any<TPR, S, R, SWI>(g, a, groups, st,
                                         std::make_integer_sequence<int, SWI ? 8 : 16>{});
}

// Register window: 2 slots (64 activation values per lane; a chunk of 16
// super-blocks = 4096 values at 8 teams per row).
template <bool SWI>
static hipError_t dispatch_xf32(const XF32Args& a, hipStream_t st) {
  if (a.nsb == 1) return run_xf32<1, 1, SWI>(a, st);
  if (a.nsb == 2) return run_xf32<2, 1, SWI>(a, st);
  if (a.nsb <= 4) return run_xf32<4, 1, SWI>(a, st);
  if (a.nsb <= 8) return run_xf32<8, 1, SWI>(a, st);
  return run_xf32<8, 2, SWI>(a, st);
}

hipError_t launch_q4k_gemv_xf32(const uint8_t* w, const float* x, int n, float* y, int out_dim,
                                int in_dim, hipStream_t stream) {
  XF32Args a{w, nullptr, x, y, nullptr, n, out_dim, in_dim / kQKK};
  return dispatch_xf32<false>(a, stream);
}

hipError_t launch_swiglu_ffn_q4k_xf32(const uint8_t* w_gate, const uint8_t* w_up,
                                      const uint8_t* w_down, const float* x, float* h, float* y,
                                      float* gu, int hidden_dim, int inter_dim,
                                      hipStream_t stream) {
  XF32Args a{w_gate, w_up, x, h, gu, hidden_dim, inter_dim, hidden_dim / kQKK};
  const hipError_t e = dispatch_xf32<true>(a, stream);
  if (e != hipSuccess) return e;
  return launch_q4k_gemv_xf32(w_down, h, inter_dim, y, hidden_dim, inter_dim, stream);
}

}  // namespace rz
