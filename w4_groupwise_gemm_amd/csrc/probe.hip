// Measurement support (built as the separate libw4probe.so, not part of the product ABI):
//   - a plain streaming read kernel: the achievable HBM read rate for a given byte count, the
//     ceiling the weight-stream numbers are compared with;
//   - a plain copy kernel of known size: FETCH_SIZE / WRITE_SIZE counters of a known traffic,
//     used to scale the counter readings of the GEMM kernels into bytes;
//   - an empty kernel: launch overhead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

// Grid-stride read with U independent 16-byte loads in flight per lane: lane i reads chunks
// i, i + S, ..., i + (U - 1) S (S = the grid's lane count) together, then moves on by U S.
template <int U>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                   uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // practically never taken; keeps the loads alive
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" int w4probe_read_u(const void* src, size_t bytes, void* sink, int grid, int unroll,
                              void* stream) {
  if (!src || !sink || (bytes & 15) || grid <= 0) return -1;
  const hipStream_t st = (hipStream_t)stream;
  const u32x4* s = (const u32x4*)src;
  hipError_t e;
  switch (unroll) {
    case 1: e = w4::launch_kernel(&read_kernel<1>, dim3(grid), dim3(256), 0, st, s, bytes / 16, (uint32_t*)sink); break;
    case 2: e = w4::launch_kernel(&read_kernel<2>, dim3(grid), dim3(256), 0, st, s, bytes / 16, (uint32_t*)sink); break;
    case 4: e = w4::launch_kernel(&read_kernel<4>, dim3(grid), dim3(256), 0, st, s, bytes / 16, (uint32_t*)sink); break;
    case 8: e = w4::launch_kernel(&read_kernel<8>, dim3(grid), dim3(256), 0, st, s, bytes / 16, (uint32_t*)sink); break;
    default: return -1;
  }
  return e == hipSuccess ? 0 : -7;
}

extern "C" int w4probe_read(const void* src, size_t bytes, void* sink, int grid, void* stream) {
  return w4probe_read_u(src, bytes, sink, grid, 1, stream);
}

extern "C" int w4probe_copy(const void* src, void* dst, size_t bytes, int grid, void* stream) {
  if (!src || !dst || (bytes & 15) || grid <= 0) return -1;
  return w4::launch_kernel(&copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                           (const u32x4*)src, (u32x4*)dst, bytes / 16) == hipSuccess ? 0 : -7;
}

extern "C" int w4probe_empty(void* stream) {
  return w4::launch_kernel(&empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream) == hipSuccess ? 0 : -7;
}
