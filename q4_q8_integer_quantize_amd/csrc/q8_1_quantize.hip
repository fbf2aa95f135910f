// q8_1_quantize.hip -- fp32 activations to Q8_1 blocks.
//
// realizar 0.8.5 src/cuda/executor/cached.rs, transformer_layer_gpu_true_dp4a,
// steps 2 and 5: the activation is quantized once and every projection that
// reads it shares the blocks.  Zero padding up to n_padded follows
// pad_and_upload_input in src/cuda/executor/layers/forward_utils.rs.
//
// An aligned group of 8 lanes owns one block (4 values per lane), so a 256-
// thread workgroup quantizes 32 blocks; the block rule is q8_1_block_group8.
#include "rz_device.h"
#include "rz_launch.h"

namespace rz {

__global__ __launch_bounds__(256) void q8_1_quantize_kernel(const float* __restrict__ x, int n,
                                                            int n_padded, long total_blocks,
                                                            uint8_t* __restrict__ out) {
  const long g = (long)blockIdx.x * (blockDim.x / 8) + (threadIdx.x >> 3);
  if (g >= total_blocks) return;   // whole 8-lane groups leave together
  const int i = threadIdx.x & 7;
  const int nb = n_padded / kQK8;
  const long t = g / nb;
  const int b = (int)(g - t * nb);
  const uint32_t bytes = (uint32_t)(total_blocks / nb) * (uint32_t)n * 4u;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)bytes, kBufferWord3);
  float v[4];
  load_block_quad(v, xr, (uint32_t)t * (uint32_t)n, b * kQK8 + 4 * i, n, true, bytes);
  float d, s;
  const uint32_t packed = q8_1_block_group8(v, d, s);
  uint8_t* blk = out + g * kQ8Bytes;
  *(uint32_t*)(blk + 8 + 4 * i) = packed;
  if (i == 0) {
    ((float*)blk)[0] = d;
    ((float*)blk)[1] = s;
  }
}

hipError_t launch_q8_1_quantize(const float* x, int n, int n_padded, int n_tokens,
                                uint8_t* out, hipStream_t stream) {
  const long total = (long)n_tokens * (n_padded / kQK8);
  const long groups_per_wg = 256 / 8;
  const unsigned grid = (unsigned)((total + groups_per_wg - 1) / groups_per_wg);
  hipLaunchKernelGGL(q8_1_quantize_kernel, dim3(grid), dim3(256), 0, stream, x, n, n_padded,
                     total, out);
  return hipGetLastError();
}

}  // namespace rz
