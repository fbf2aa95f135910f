// stream_read.hip -- a plain streaming read of a device buffer: the bandwidth
// a kernel that only reads the same bytes reaches on this part, reported next
// to the GEMV's as its practical ceiling.  Not part of the GEMV path and not
// in librz.so; it is built into a library of its own for the benchmark.
//
// Every 16-byte chunk is loaded once (non-temporal, U chunks a thread in
// flight per step of a grid-stride loop) and folded into one word per thread;
// the word is stored only when it equals a constant the data never folds to,
// so the loads stay live and nothing is written.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

typedef uint32_t rd_u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const rd_u32x4* __restrict__ p, long n16,
                                                          uint32_t* __restrict__ sink) {
  const long stride = (long)gridDim.x * 256 * U;
  uint32_t acc = 0;
  for (long i = (long)blockIdx.x * 256 * U + threadIdx.x; i < n16; i += stride) {
    rd_u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long j = i + (long)u * 256;
      v[u] = j < n16 ? __builtin_nontemporal_load(p + j) : (rd_u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

// Reads bytes (a multiple of 16) at p, 16-byte aligned, with `grid`
// workgroups of 256 threads; sink is 1 KiB of device memory.  Returns 0, or
// -1 for invalid arguments, or the HIP error code of the launch.
extern "C" int rz_stream_read(const void* p, size_t bytes, void* sink, int grid, void* stream) {
  if (p == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 ||
      ((uintptr_t)p & 15u) != 0 || grid < 1 || grid > 65536)
    return -1;
  hipLaunchKernelGGL((stream_read_kernel<4>), dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const rd_u32x4*)p, (long)(bytes / 16), (uint32_t*)sink);
  return (int)hipGetLastError();
}
