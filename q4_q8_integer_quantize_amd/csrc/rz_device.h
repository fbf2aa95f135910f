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

// Sum over aligned groups of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, W);
  return v;
}
template <int W>
__device__ __forceinline__ int group_sum_i(int v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, W);
  return v;
}
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, W));
  return v;
}

// One Q8_1 block quantized by an aligned group of 8 lanes; lane i (0..7) holds
// values 4i..4i+3.  Returns this lane's four codes packed little-endian and
// sets d and s (identical in all 8 lanes).  The rule: amax = max|x| (exact),
// d = amax / 127 (correctly rounded fp32 division), q = rint(x / d) (fp32
// division, ties to even), s = d * float(sum q); amax == 0 gives zeros.
__device__ __forceinline__ uint32_t q8_1_block_group8(const float v[4], float& d, float& s) {
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  amax = group_max<8>(amax);
  d = amax / 127.0f;
  uint32_t packed = 0;
  int sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int q = 0;
    if (amax != 0.0f) {
      float r = rintf(v[k] / d);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      q = (int)r;
    }
    sum += q;
    packed |= ((uint32_t)(q & 0xff)) << (8 * k);
  }
  sum = group_sum_i<8>(sum);
  s = d * (float)sum;
  if (amax == 0.0f) { d = 0.0f; s = 0.0f; }
  return packed;
}

}  // namespace rz
