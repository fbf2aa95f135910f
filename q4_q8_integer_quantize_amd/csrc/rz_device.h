// rz_device.h -- device-side building blocks shared by the librz kernels.
//
// Block geometry (GGML layouts, see include/rz.h):
//   Q8_1 : 40 B  = f32 d | f32 s | i8 q[32]
//   Q4_K : 144 B = f16 d | f16 dmin | u8 scales[12] | u8 qs[128]   (256 values)
//   Q4_0 : 18 B  = f16 d | u8 qs[16]                               (32 values)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rz {

constexpr int kWave = 64;
constexpr int kQK8 = 32;
constexpr int kQ8Bytes = 40;
constexpr int kQKK = 256;
constexpr int kQ4KBytes = 144;
constexpr int kQK40 = 32;
constexpr int kQ40Bytes = 18;
// Raw buffer descriptor word 3 (data format 32, no swizzle) for gfx9 parts.
constexpr int kBufferWord3 = 0x00020000;

// 16-byte vector whose pointer only promises 4-byte alignment; gfx9 global
// loads accept dword-aligned addresses for multi-dword accesses.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int dot4(int a, int b, int acc) {
  // v_dot4_i32_i8: four signed int8 products accumulated into int32.
  // Nibbles 0..15 are valid non-negative int8 values, so the signed form
  // serves the unsigned-nibble x signed-code product exactly.
  return __builtin_amdgcn_sdot4(a, b, acc, false);
}

__device__ __forceinline__ uint32_t bits(uint32_t v, uint32_t off, uint32_t len) {
  // field of `len` bits at `off`; len == 0 yields 0
  return (v >> off) & ((1u << len) - 1u);
}

__device__ __forceinline__ float f16_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// v & m, opaque to the compiler's known-bits analysis.  With a nibble mask
// visible, a byte conversion of the result folds into a 4-bit extract plus a
// byte-0 conversion (two instructions per weight); behind this AND each byte
// converts with one v_cvt_f32_ubyte{0..3}.  Used by the fp32-activation dots.
__device__ __forceinline__ uint32_t opaque_and(uint32_t v, uint32_t m) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(v), "v"(m));
  return r;
}

// DPP lane exchange within rows of 16 lanes (control words: quad_perm
// [1,0,3,2] = 0xB1 is lane^1, [2,3,0,1] = 0x4E is lane^2, row_half_mirror
// 0x141 swaps the two quads of each group of 8, row_mirror 0x140 the two
// groups of 8 of a row, row_bcast 0x142 / 0x143 broadcast lane 15 / 31).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL, ROW_MASK>(__builtin_bit_cast(int, v)));
}

// Sum over aligned groups of W lanes (W a power of two, 1..64) with DPP.  The
// full sum is valid in the LAST lane of each group (for W <= 16 in every lane).
template <int W>
__device__ __forceinline__ float group_sum_dpp(float v) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
  if constexpr (W >= 2) v += dpp_f<0xB1>(v);          // lane ^ 1
  if constexpr (W >= 4) v += dpp_f<0x4E>(v);          // lane ^ 2
  if constexpr (W >= 8) v += dpp_f<0x141>(v);         // quads of an 8
  if constexpr (W >= 16) v += dpp_f<0x140>(v);        // 8-groups of a row
  if constexpr (W >= 32) v += dpp_f<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
  if constexpr (W >= 64) v += dpp_f<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
  return v;
}

// Four consecutive activation values x[base + idx .. base + idx + 3], read as
// single dwords through a raw buffer descriptor that spans exactly x (`bytes`).
// Values at idx + k >= n, or of an inactive block, take the offset `bytes`,
// which the hardware range check turns into 0: no branch and no clamping, so
// the loads of several blocks stay in flight together.
__device__ __forceinline__ void load_block_quad(float v[4], __amdgpu_buffer_rsrc_t xr,
                                                uint32_t base, int idx, int n, bool active,
                                                uint32_t bytes) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = idx + k;
    const uint32_t off = (active && j < n) ? (base + (uint32_t)j) * 4u : bytes;
    v[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0));
  }
}

// One Q8_1 block quantized by an aligned group of 8 lanes; lane i (0..7) holds
// values 4i..4i+3.  Returns this lane's four codes packed little-endian and
// sets d and s (identical in all 8 lanes).  The rule: amax = max|x| (exact),
// d = amax / 127 (correctly rounded fp32 division), q = rint(x / d) (the
// correctly rounded fp32 quotient, ties to even), s = d * float(sum q);
// d == 0 (amax == 0, or so small that amax / 127 rounds to 0) gives zeros.
// Branch-free: the 8-lane max and sum run on DPP, and a zero block takes its
// zero codes through a zero reciprocal (its quotients have no value).
__device__ __forceinline__ uint32_t q8_1_block_group8(const float v[4], float& d, float& s) {
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  // the 8-lane maximum on bit patterns: non-negative floats order as their
  // bit patterns do as integers, and an integer max takes the DPP operand
  {
    int ai = __builtin_bit_cast(int, amax);
    ai = max(ai, dpp_i<0xB1>(ai));
    ai = max(ai, dpp_i<0x4E>(ai));
    ai = max(ai, dpp_i<0x141>(ai));
    amax = __builtin_bit_cast(float, ai);
  }
  // Every quotient here is the correctly rounded one, computed without a
  // division (Markstein's theorem): with y the correctly rounded reciprocal of
  // the divisor b, q0 = a*y is within an ulp of a/b, the residual a - q0*b is
  // exact in one fma, and q0 + residual*y rounds to exactly RN(a/b).
  // d = RN(amax / 127) this way, with y = RN(1/127) a constant: equal to the
  // division for every non-negative float, denormals included.
  constexpr float kInv127 = 1.0f / 127.0f;
  {
    const float q0 = amax * kInv127;
    d = __builtin_fmaf(__builtin_fmaf(-q0, 127.0f, amax), kInv127, q0);
  }
  // amax == 0, and amax of at most 63 * 2^-149, where d rounds to 0 and the
  // quotients have no value: the block of zeros
  const bool zero = d == 0.0f;
  // The four v/d: y is the hardware reciprocal after one Newton step.  From
  // any start within an ulp that step lands on RN(1/d), except for the
  // all-ones significand from its lower neighbour (Markstein's exception); on
  // this GPU the reciprocal plus the step equals RN(1/d) for every normal d
  // below 2^126, and d here is at most 2^121.  The quotients equal the
  // division for 2^30 sampled pairs.  A block with amax < 2^-60 is scaled by
  // 2^64 first (exact), so that d, its reciprocal and every residual stay
  // normal.
  const float sc = amax < 0x1p-60f ? 0x1p64f : 1.0f;
  const float ds = d * sc;
  const float y0 = __builtin_amdgcn_rcpf(ds);
  // a zero block takes y = 0, so that every quotient is 0
  const float y = zero ? 0.0f : __builtin_fmaf(__builtin_fmaf(-ds, y0, 1.0f), y0, y0);
  uint32_t packed = 0;
  int sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float xs = v[k] * sc;
    const float q0 = xs * y;
    float r = rintf(__builtin_fmaf(__builtin_fmaf(-q0, ds, xs), y, q0));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    const int q = (int)r;
    sum += q;
    packed |= ((uint32_t)(q & 0xff)) << (8 * k);
  }
  sum += dpp_i<0xB1>(sum);
  sum += dpp_i<0x4E>(sum);
  sum += dpp_i<0x141>(sum);
  s = d * (float)sum;
  return packed;
}

}  // namespace rz
