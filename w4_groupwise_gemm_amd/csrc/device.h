// Device-side building blocks shared by the kernels: vector types, wait and register helpers,
// the in-register decode of packed 4/5-bit codes, the matrix-core steps and the epilogues.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "layout.h"

namespace w4dev {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_ADD = 2 };

__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// A 32-bit register that holds the constant (keeps v_and_or_b32 legal: one literal or SGPR).
__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// Wait until at most N vector-memory operations of this wave are outstanding (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence.  The fence that __syncthreads() adds would wait for
// every outstanding load of the wave, including the ones meant to stay in flight; the waits are
// explicit instead (producers: vmcnt for their own loads; consumers: lgkmcnt for their LDS
// reads).  The "memory" clobber keeps the compiler from moving memory operations across it.
__device__ __forceinline__ void arrive_wait() {
  // lgkmcnt(0) as a builtin, so that the compiler's own wait insertion knows every earlier LDS
  // read has completed; the barrier itself as volatile asm with a memory clobber
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63 (no wait), expcnt 7, lgkmcnt 0
  asm volatile("s_barrier" ::: "memory");
}

// (a & mask) | c in one v_and_or_b32 (the compiler can otherwise form and + and + or3)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(c));
  return r;
}

// Biased fp16 pairs of packed dword J: 1024 + q (slots 0,1 and 4,5) and 1024 + 16 q (slots 2,3
// and 6,7).  OR-ing a 4-bit field into the mantissa of fp16 1024.0 (magic = 0x64006400) gives
// 1024 + q exactly, with no integer-to-float conversion (the "magic-bias" decode of the
// ninfer-3080 performance notes, "What changed", "Permuted k order", here in fp16).  For 5-bit
// codes bit 4 comes from the lane's high-plane word at mantissa bit 4 (resp. 8), one shift and
// one mask-or per pair given the packed high-plane bit positions.
template <int BITS, int J>
__device__ __forceinline__ void wbiased(uint32_t w, uint32_t hiw, uint32_t magic, uint32_t u[4]) {
  const uint32_t w8 = w >> 8;
  u[0] = and_or(w, 0x000F000Fu, magic);
  u[1] = and_or(w, 0x00F000F0u, magic);
  u[2] = and_or(w8, 0x000F000Fu, magic);
  u[3] = and_or(w8, 0x00F000F0u, magic);
  if constexpr (BITS == 5) {
    constexpr int t = (J == 0 ? 0 : J == 1 ? 2 : J == 2 ? 8 : 10);
    uint32_t x1, x2;
    if constexpr (t <= 3) {
      x1 = hiw << (4 - t);
      x2 = hiw << (3 - t);
    } else {
      x1 = hiw >> (t - 4);
      x2 = hiw >> (t - 3);
    }
    u[0] = and_or(x1, 0x00100010u, u[0]);
    u[1] = and_or(x1, 0x01000100u, u[1]);
    u[2] = and_or(x2, 0x00100010u, u[2]);
    u[3] = and_or(x2, 0x01000100u, u[3]);
  }
}

__device__ __forceinline__ f16x8 cat8(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  const f16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const f16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Broadcast the fp16 value in the low (H == 0) or high (H == 1) half of a packed pair.
template <int H>
__device__ __forceinline__ f16x2 splat(uint32_t pair) {
  const f16x2 p = as_h2(pair);
  return __builtin_shufflevector(p, p, H, H);
}

// 16x16x32 fp16 matrix-core step, fp32 accumulate.  A lane l supplies A row l%16 and B column
// l%16, k slots 8*(l/16)..+7; the lane then holds D rows 4*(l/16)+i, column l%16, i = 0..3.
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 32x32x16 fp16 matrix-core step, fp32 accumulate.  A lane l supplies A row l%32 and B column
// l%32, k slots 8*(l/32)..+7; the lane then holds D rows 8*(v/4) + 4*(l/32) + v%4 in register
// v (v = 0..15), column l%32.
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + expf(-a)); }

__device__ __forceinline__ float bf16_value(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t bf16_bits(float f) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Epilogue of one output quad: 4 consecutive output columns n..n+3 of token t (the caller
// guarantees t < T and n + 3 < ldo).  fp16 activations: out = fp16(v) / fp16(silu(v) * up) /
// fp16(v + res).  bf16 activations (a.xexp set): the sums were formed from X[t] * 2^-e, so they
// are scaled by 2^e first, the residual is bf16, and the result is rounded to bf16.
template <int EPI>
__device__ __forceinline__ void store_quad(const w4::KArgs& a, int t, int n, f32x4 v, f32x4 up) {
  const size_t off = (size_t)t * a.ldo + n;
  if (a.xexp) {
    const int e = a.xexp[t];
    uint16_t h[4];
    const uint16_t* r16 = reinterpret_cast<const uint16_t*>(a.res);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float y = ldexpf(v[i], e);
      if constexpr (EPI == EPI_ADD) y = y + bf16_value(r16[off + i]);
      if constexpr (EPI == EPI_SWIGLU) y = silu(y) * ldexpf(up[i], e);
      h[i] = bf16_bits(y);
    }
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + off) =
        u32x2{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
    return;
  }
  f16x4 h;
  if constexpr (EPI == EPI_ADD) {
    const f16x4 r = *reinterpret_cast<const f16x4*>(a.res + off);
    h[0] = (f16)(v[0] + (float)r[0]);
    h[1] = (f16)(v[1] + (float)r[1]);
    h[2] = (f16)(v[2] + (float)r[2]);
    h[3] = (f16)(v[3] + (float)r[3]);
  } else if constexpr (EPI == EPI_SWIGLU) {
    h[0] = (f16)(silu(v[0]) * up[0]);
    h[1] = (f16)(silu(v[1]) * up[1]);
    h[2] = (f16)(silu(v[2]) * up[2]);
    h[3] = (f16)(silu(v[3]) * up[3]);
  } else {
    h[0] = (f16)v[0];
    h[1] = (f16)v[1];
    h[2] = (f16)v[2];
    h[3] = (f16)v[3];
  }
  *reinterpret_cast<f16x4*>(a.out + off) = h;
}

// One output element (token t, column n), same rules.
template <int EPI>
__device__ __forceinline__ void store_one(const w4::KArgs& a, int t, int n, float v, float up) {
  const size_t off = (size_t)t * a.ldo + n;
  if (a.xexp) {
    const int e = a.xexp[t];
    float y = ldexpf(v, e);
    if constexpr (EPI == EPI_ADD) y = y + bf16_value(reinterpret_cast<const uint16_t*>(a.res)[off]);
    if constexpr (EPI == EPI_SWIGLU) y = silu(y) * ldexpf(up, e);
    reinterpret_cast<uint16_t*>(a.out)[off] = bf16_bits(y);
    return;
  }
  if constexpr (EPI == EPI_ADD) {
    a.out[off] = (f16)(v + (float)a.res[off]);
  } else if constexpr (EPI == EPI_SWIGLU) {
    a.out[off] = (f16)(silu(v) * up);
  } else {
    a.out[off] = (f16)v;
  }
}

}  // namespace w4dev
