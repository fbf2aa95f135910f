// stream_read.hip -- a plain streaming read of a device buffer: the bandwidth
// a kernel that only reads the same bytes reaches on this part, reported next
// to the GEMV's as its practical ceiling.  Not part of the GEMV path and not
// in librz.so; it is built into a library of its own for the benchmark.
//
// Every 16-byte chunk is loaded once (non-temporal) and folded into one word
// per thread; the word is stored only when it equals a constant the data never
// folds to, so the loads stay live and nothing is written.  Two shapes: a
// grid-stride loop with U chunks a thread in flight per step, and a one-shot
// grid in which every thread loads its U chunks and exits (the fastest shape
// found for a 33 MB read on MI355X: two chunks a thread).
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

template <int U>
__global__ __launch_bounds__(256) void stream_read_once_kernel(const rd_u32x4* __restrict__ p, long n16,
                                                               uint32_t* __restrict__ sink) {
  const long base = (long)blockIdx.x * 256 * U + threadIdx.x;
  rd_u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const long j = base + (long)u * 256;
    v[u] = j < n16 ? __builtin_nontemporal_load(p + j) : (rd_u32x4){0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

// The one-shot shape: ceil(bytes / (4096 u)) workgroups of 256 threads, each
// thread loading u (1, 2, 4 or 8) 16-byte chunks.  Same arguments and returns
// as rz_stream_read otherwise.
extern "C" int rz_stream_read_once(const void* p, size_t bytes, void* sink, int u, void* stream) {
  if (p == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 ||
      ((uintptr_t)p & 15u) != 0 || (u != 1 && u != 2 && u != 4 && u != 8))
    return -1;
  const long n16 = (long)(bytes / 16);
  const long grid = (n16 + 256L * u - 1) / (256L * u);
  if (grid > 0x7fffffffL) return -1;
  const hipStream_t st = (hipStream_t)stream;
  switch (u) {
    case 1: hipLaunchKernelGGL((stream_read_once_kernel<1>), dim3((unsigned)grid), dim3(256), 0, st, (const rd_u32x4*)p, n16, (uint32_t*)sink); break;
    case 2: hipLaunchKernelGGL((stream_read_once_kernel<2>), dim3((unsigned)grid), dim3(256), 0, st, (const rd_u32x4*)p, n16, (uint32_t*)sink); break;
    case 4: hipLaunchKernelGGL((stream_read_once_kernel<4>), dim3((unsigned)grid), dim3(256), 0, st, (const rd_u32x4*)p, n16, (uint32_t*)sink); break;
    default: hipLaunchKernelGGL((stream_read_once_kernel<8>), dim3((unsigned)grid), dim3(256), 0, st, (const rd_u32x4*)p, n16, (uint32_t*)sink); break;
  }
  return (int)hipGetLastError();
}
