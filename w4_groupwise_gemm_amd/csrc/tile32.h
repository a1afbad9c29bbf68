// Building blocks of the 32x32x16 matrix-core kernels (wide and narrow paths): buffer
// resources, the in-register dequantisation of packed dwords, the lane map of a 32-row tile
// pair, the swizzled activation tile in LDS and the epilogue of one 32 x 32 accumulator.
#pragma once
#include "device.h"
#include "kernels.h"

namespace w4 {
namespace t32 {

using namespace w4dev;
using w4layout::block_bytes;

constexpr int kXCD = 8;  // gfx950 (MI350 series): 8 accelerator complex dies, round-robin dispatch

// fp16 weights (q - z) * s of packed dword J (8 k slots of one row).  FAST: z is an integer,
// so 1024 + z and 64 + z are exact and one packed add (or fma) removes bias and zero-point.
template <int BITS, int J, bool FAST>
__device__ __forceinline__ f16x8 wfrag(uint32_t w, uint32_t hiw, uint32_t magic, uint32_t zp,
                                       uint32_t sp) {
  uint32_t u[4];
  wbiased<BITS, J>(w, hiw, magic, u);
  const f16x2 z2 = splat<(J >> 1)>(zp), s2 = splat<(J >> 1)>(sp);
  const f16x2 c16th = {(f16)0.0625f, (f16)0.0625f};
  const f16x2 c1024 = {(f16)1024.0f, (f16)1024.0f}, c64 = {(f16)64.0f, (f16)64.0f};
  if constexpr (FAST) {
    const f16x2 b0 = -(z2 + c1024), b1 = -(z2 + c64);
    return cat8((as_h2(u[0]) + b0) * s2, (as_h2(u[1]) * c16th + b1) * s2, (as_h2(u[2]) + b0) * s2,
                (as_h2(u[3]) * c16th + b1) * s2);
  } else {
    return cat8(((as_h2(u[0]) - c1024) - z2) * s2, ((as_h2(u[1]) * c16th - c64) - z2) * s2,
                ((as_h2(u[2]) - c1024) - z2) * s2, ((as_h2(u[3]) * c16th - c64) - z2) * s2);
  }
}

// Buffer resource over `bytes` bytes at `base` (gfx9 raw buffer, 32-bit offsets; reads past
// the end return zero instead of faulting).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

struct Rsrcs {
  __amdgpu_buffer_rsrc_t x, w, s, z;
};

// Lane-constant parts of the code addresses.
struct LaneMap {
  int slot16[2];  // byte offset of the lane's 16-byte code slot in a block, sets 0 and 1
  int th;         // tile of the pair (0 / 1) this lane reads
  int szoff;      // byte offset of the lane's scale / zero-point pair in a (tile, k-block) block
};

// The lane's source lane groups S + 2 (lane / 32), S = 0, 1, fall in one half of the lane
// groups, so one scale / zero-point pair serves both code sets for every group size.
__device__ __forceinline__ LaneMap lane_map(const KArgs& a, int lane) {
  LaneMap m;
  m.th = (lane >> 4) & 1;
  m.szoff = 4 * sz_lane_word(a, lane & 15, 2 * (lane >> 5));
#pragma unroll
  for (int s = 0; s < 2; ++s) m.slot16[s] = ((lane & 15) + 16 * (s + 2 * (lane >> 5))) * 16;
  return m;
}

// A-operand words of one 32-row pair and one k-block, for this lane.  Set S (0 / 1) is the
// 16-byte load of k-steps (j, S), j = 0..3; the lane's row is pair row lane % 32, its k half
// h = lane / 32.  In packed terms: 16-lane group (lane / 16) reads tile a, b, a, b of the pair,
// and the source lane inside that tile is lane % 16 + 16 (S + 2 h), whose k slots are
// 64 (j / 2) + 16 (S + 2 h) + 8 (j % 2) + e.
template <int BITS>
struct PairCodes {
  u32x4 cw[2];
  uint32_t hw[2];   // high-bit planes (5-bit only)
  uint32_t sp, zp;  // this lane's row: fp16 scale / zero-point pairs (groups 0, 1 of the block)
};

// Every offset below is lane-dependent, so it goes in the lane operand; the tile index is
// clamped to the last tile (an odd tile count leaves the second tile of the last pair empty:
// its rows are computed from the clamped tile and never stored).
template <int BITS>
__device__ __forceinline__ void load_pair(PairCodes<BITS>& c, const Rsrcs& R, const KArgs& a,
                                          const LaneMap& m, int pair, int ntiles, int kb) {
  constexpr int BLK = block_bytes(BITS);
  const int tile = min(2 * pair + m.th, ntiles - 1);
  const int bi = tile * a.KB + kb;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    c.cw[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.w, bi * BLK + m.slot16[s], 0, 0));
    if constexpr (BITS == 5)
      c.hw[s] = __builtin_amdgcn_raw_buffer_load_b32(R.w, bi * BLK + 1024 + m.slot16[s] / 4, 0, 0);
    else
      c.hw[s] = 0;
  }
  c.sp = __builtin_amdgcn_raw_buffer_load_b32(R.s, bi * 4 * a.szw + m.szoff, 0, 0);
  c.zp = __builtin_amdgcn_raw_buffer_load_b32(R.z, bi * 4 * a.szw + m.szoff, 0, 0);
}

// Direct-to-LDS load of the activation tile of k-block kb: BN token rows x 16 chunks of 16 B.
// One instruction moves 4 token rows (64 lanes x 16 B, contiguous in LDS); lane L of it takes
// row r0 + L/16 and stores LDS chunk L%16, which holds source chunk (L%16) ^ (row & 15).  The
// swizzled part of the lane offset depends on (r0 & 15) / 4 only (four precomputed offsets);
// the row and column part is added per instruction.  The whole offset goes in the lane
// (range-checked) operand: token rows beyond T and columns past the end of the last row lie
// past the end of the buffer resource and read as zero.  Columns beyond K inside the buffer
// (half-empty last block) read the next row; those k slots are skipped by the math.
template <int BN>
__device__ __forceinline__ void load_x_lds(const Rsrcs& R, const KArgs& a, char* xs,
                                           const int (&voff)[4], int tok0, int kb, int wave) {
  constexpr int PER_WAVE = BN / 16;  // instructions per wave
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int r0 = (wave * PER_WAVE + i) * 4;
    const int rowoff = ((tok0 + r0) * a.K + kb * 128) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        R.x, (__attribute__((address_space(3))) void*)(xs + r0 * 256), 16,
        voff[(r0 & 15) >> 2] + rowoff, 0, 0, 0);
  }
}

// B lane l of step (J, S) = step I = 2 J + S, token tile tt: token row 32 tt + l%32,
// k = 64 (J/2) + 16 (S + 2 h) + 8 (J%2) + e,
// i.e. LDS chunk c = 8 (J/2) + (J%2) + 2 S + 4 h stored at c ^ (row & 15).  With
// bsw = row * 256 + 16 ((4 h) ^ (row & 15)) and the constant part of c disjoint from 4 h in
// bits, the slot is bsw ^ 16 C.
template <int I>
__device__ __forceinline__ f16x8 load_b1(const char* xs, int bsw, int tt) {
  constexpr int J = I >> 1, S = I & 1;
  constexpr int C = 8 * (J >> 1) + (J & 1) + 2 * S;
  return *reinterpret_cast<const f16x8*>(xs + (bsw ^ (16 * C)) + tt * 32 * 256);
}
// The same for NTT token tiles.
template <int NTT, int I>
__device__ __forceinline__ void load_b(const char* xs, int bsw, f16x8 (&B)[NTT]) {
  constexpr int J = I >> 1, S = I & 1;
  constexpr int C = 8 * (J >> 1) + (J & 1) + 2 * S;
  const char* xb = xs + (bsw ^ (16 * C));
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) B[tt] = *reinterpret_cast<const f16x8*>(xb + tt * 32 * 256);
}

// Epilogue of one 32 x 32 accumulator: pair `pair`, tokens tok .. tok + 31.  Lane l holds token
// tok + l%32 and, in registers 4q .. 4q+3, pair rows 8q + 4 (l/32) + 0..3 (4 consecutive output
// columns).  SwiGLU pairs are (gate tile, up tile): gate row r sits in register v and the up
// row of the same output column r in register v + 8 of the same lane.
template <int EPI>
__device__ __forceinline__ void store_pair(const KArgs& a, const f32x16& v, int pair, int tok,
                                           int ntiles, int lane) {
  const int t = tok + (lane & 31);
  if (t >= a.T || 2 * pair >= ntiles) return;
  const int h = lane >> 5;
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
      store_quad<EPI>(a, t, 16 * pair + 8 * q + 4 * h,
                      f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]},
                      f32x4{v[8 + 4 * q], v[9 + 4 * q], v[10 + 4 * q], v[11 + 4 * q]});
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q >= 2 && 2 * pair + 1 >= ntiles) break;  // odd tile count: no second tile
      store_quad<EPI>(a, t, 32 * pair + 8 * q + 4 * h,
                      f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]}, f32x4{});
    }
  }
}

}  // namespace t32
}  // namespace w4
