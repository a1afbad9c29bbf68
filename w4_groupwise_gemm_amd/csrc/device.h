// Device-side building blocks shared by the kernels: vector types, the in-register decode of
// packed 4/5-bit codes, the fp16 dequantisation, the matrix-core step and the epilogues.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Exact codes q as four fp16 pairs -- slots (0,1), (2,3), (4,5), (6,7) -- of packed dword J.
// OR-ing a 4-bit field into the mantissa of fp16 1024.0 (0x6400) gives 1024 + q exactly
// (bits 0..3) or 1024 + 16 q (bits 4..7); one packed add or fma removes the bias.  For 5-bit
// codes bit 4 is OR-ed in from the lane's high-plane word at mantissa bit 4 (resp. 8), which
// the high-plane bit positions of the packed layout make one shift + one mask-or per pair.
// This is the "magic-bias" decode the ninfer-3080 performance notes mention ("What changed",
// "Permuted k order"), done here with fp16 instead of bf16 and without integer-to-float ops.
template <int BITS, int J>
__device__ __forceinline__ void decode_q(uint32_t w, uint32_t hiw, f16x2 q[4]) {
  constexpr uint32_t kMagic = 0x64006400u;  // fp16 1024.0 in both halves
  const uint32_t w8 = w >> 8;
  uint32_t u0 = (w & 0x000F000Fu) | kMagic;   // 1024 + q      (slots 0, 1)
  uint32_t u1 = (w & 0x00F000F0u) | kMagic;   // 1024 + 16 q   (slots 2, 3)
  uint32_t u2 = (w8 & 0x000F000Fu) | kMagic;  // 1024 + q      (slots 4, 5)
  uint32_t u3 = (w8 & 0x00F000F0u) | kMagic;  // 1024 + 16 q   (slots 6, 7)
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
    u0 |= x1 & 0x00100010u;
    u1 |= x1 & 0x01000100u;
    u2 |= x2 & 0x00100010u;
    u3 |= x2 & 0x01000100u;
  }
  const f16x2 c1024 = {(f16)1024.0f, (f16)1024.0f};
  const f16x2 c64 = {(f16)64.0f, (f16)64.0f};
  const f16x2 c16th = {(f16)0.0625f, (f16)0.0625f};
  q[0] = as_h2(u0) - c1024;
  q[1] = as_h2(u1) * c16th - c64;
  q[2] = as_h2(u2) - c1024;
  q[3] = as_h2(u3) * c16th - c64;
}

__device__ __forceinline__ f16x8 cat8(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  const f16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const f16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// fp16 weights w = (q - z) * s for the 8 slots of packed dword J (one rounding when z is an
// integer: q - z is then exact in fp16).  z2 / s2 hold the group's zero-point / scale twice.
template <int BITS, int J>
__device__ __forceinline__ f16x8 dequant8(uint32_t w, uint32_t hiw, f16x2 z2, f16x2 s2) {
  f16x2 q[4];
  decode_q<BITS, J>(w, hiw, q);
  return cat8((q[0] - z2) * s2, (q[1] - z2) * s2, (q[2] - z2) * s2, (q[3] - z2) * s2);
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

// Epilogue of one output quad: 4 consecutive output columns n..n+3 of token t.
// out / res are fp16 [T][ldo]; the caller guarantees t < T and n + 3 < ldo.
template <int EPI>
__device__ __forceinline__ void store_quad(f16* out, const f16* res, size_t off, f32x4 v,
                                           f32x4 up) {
  f16x4 h;
  if constexpr (EPI == EPI_ADD) {
    const f16x4 r = *reinterpret_cast<const f16x4*>(res + off);
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
  *reinterpret_cast<f16x4*>(out + off) = h;
}

template <int EPI>
__device__ __forceinline__ void store_one(f16* out, const f16* res, size_t off, float v, float up) {
  if constexpr (EPI == EPI_ADD) {
    out[off] = (f16)(v + (float)res[off]);
  } else if constexpr (EPI == EPI_SWIGLU) {
    out[off] = (f16)(silu(v) * up);
  } else {
    out[off] = (f16)v;
  }
}

}  // namespace w4dev
