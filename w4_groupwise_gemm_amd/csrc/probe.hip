// Measurement support (built as the separate libw4probe.so, not part of the product ABI):
//   - a plain streaming read kernel: the achievable HBM read rate for a given byte count, the
//     ceiling the weight-stream numbers are compared with;
//   - a plain copy kernel of known size: FETCH_SIZE / WRITE_SIZE counters of a known traffic,
//     used to scale the counter readings of the GEMM kernels into bytes;
//   - a broadcast read: every workgroup reads the same small buffer (it stays in L2), the rate at
//     which compute units can pull an activation matrix that each of them needs whole;
//   - an LDS read loop: the shared-memory read rate per compute unit at a given number of waves;
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

// Every workgroup (4 waves) reads all n16 16-byte chunks of src, 4 in flight per lane: into
// registers (DMA = false) or straight into LDS with buffer_load ... lds (DMA = true; a 16 KB
// region per wave, overwritten, as an activation ring refill does).  Chunks past n16 read zero
// through the range-checked buffer.
template <bool DMA>
__global__ __launch_bounds__(256) void bcast_kernel(const u32x4* __restrict__ src, int n16,
                                                    uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) char lds[DMA ? 4 * 16384 : 16];
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4*>(src), (short)0, n16 * 16, 0x00020000);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t acc = 0;
  for (int i = wave * 64; i < n16; i += 4 * 256) {
    if constexpr (DMA) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + wave * 16384 + u * 1024),
                                                 16, (i + u * 256 + lane) * 16, 0, 0, 0);
    } else {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (i + u * 256 + lane) * 16, 0, 0));
#pragma unroll
      for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
  }
  if constexpr (DMA) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    acc = reinterpret_cast<const uint32_t*>(lds)[threadIdx.x];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // practically never taken
}

// Each lane reads 16-byte chunks of a 32 KB LDS array, 8 independent reads per iteration, lanes
// of a wave on consecutive chunks (no bank conflicts).
__global__ __launch_bounds__(1024) void lds_read_kernel(int iters, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) u32x4 buf[2048];
  for (int i = threadIdx.x; i < 2048; i += blockDim.x) buf[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int l = threadIdx.x & 63;
  int base = (threadIdx.x >> 6) * 64;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= buf[(base + l + 256 * u) & 2047];
    base = (base + 64) & 2047;
  }
  const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (r == 0x9E3779B9u) sink[0] = r;
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

// Broadcast read: grid workgroups each read the first `bytes` of src (bytes < 1 GiB); dma != 0
// loads straight into LDS.
extern "C" int w4probe_bcast(const void* src, size_t bytes, void* sink, int grid, int dma,
                             void* stream) {
  if (!src || !sink || (bytes & 15) || bytes >= (1ull << 30) || grid <= 0) return -1;
  const hipStream_t st = (hipStream_t)stream;
  const int n16 = (int)(bytes / 16);
  const hipError_t e = dma ? w4::launch_kernel(&bcast_kernel<true>, dim3(grid), dim3(256), 0, st, (const u32x4*)src, n16, (uint32_t*)sink)
                           : w4::launch_kernel(&bcast_kernel<false>, dim3(grid), dim3(256), 0, st, (const u32x4*)src, n16, (uint32_t*)sink);
  return e == hipSuccess ? 0 : -7;
}

// LDS read loop: grid workgroups of `threads` lanes (a multiple of 64, at most 1024), iters
// iterations of 8 16-byte reads per lane.
extern "C" int w4probe_lds(int iters, void* sink, int grid, int threads, void* stream) {
  if (!sink || iters <= 0 || grid <= 0 || threads <= 0 || threads > 1024 || threads % 64) return -1;
  return w4::launch_kernel(&lds_read_kernel, dim3(grid), dim3(threads), 0, (hipStream_t)stream, iters,
                           (uint32_t*)sink) == hipSuccess ? 0 : -7;
}

extern "C" int w4probe_empty(void* stream) {
  return w4::launch_kernel(&empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream) == hipSuccess ? 0 : -7;
}
