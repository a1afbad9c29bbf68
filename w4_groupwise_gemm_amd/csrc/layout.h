// Packed weight layout constants and index maps, shared by the host repacker and the device
// kernels (both sides of the library must agree on them; the oracle does not use them).
// The byte-level specification is in include/w4gemm.h.
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define W4_HD __host__ __device__
#else
#define W4_HD
#endif

namespace w4layout {

constexpr int kRowTile = 16;   // rows per packed row tile (one matrix-core A tile)
constexpr int kBlockK = 128;   // columns per packed k-block
constexpr int kGroup = 64;     // columns per scale/zero group of the measured format

W4_HD constexpr int num_kblocks(int K) { return (K + kBlockK - 1) / kBlockK; }
W4_HD constexpr int block_bytes(int bits) { return bits == 5 ? 1280 : 1024; }

// Group sizes the packed layout supports, and K's granularity for each.
W4_HD constexpr bool group_ok(int group) { return group == 32 || group == 64 || group == 128; }
W4_HD constexpr int k_multiple(int group) { return group == 128 ? 128 : 64; }
// 32-bit scale (or zero-point) words per (row tile, k-block): one fp16 pair per row, and for
// groups of 32 one pair per row and lane-group half.  Groups of 128 use the 64-column layout
// with both halves of a pair equal, so every kernel reads them as groups of 64.
W4_HD constexpr int sz_words(int group) { return group == 32 ? 32 : 16; }
// Word, inside a (row tile, k-block) block, of the pair that row r needs when its codes come
// from lane group g (columns 16 g .. 16 g + 15 of each 64-column half): halves h = 0, 1 hold
// the groups of the two halves.
W4_HD constexpr int sz_word(int group, int r, int g) { return group == 32 ? 16 * (g >> 1) + r : r; }

// Column k held by slot e (0..7) of dword j (0..3) of a lane in lane group g (0..3).
W4_HD constexpr int slot_k(int kb, int g, int j, int e) {
  return kBlockK * kb + 64 * (j >> 1) + 16 * g + 8 * (j & 1) + e;
}
// Bit position of slot e's low four bits inside its dword.
W4_HD constexpr int lo_bit(int e) { return 4 * (e >> 1) + 16 * (e & 1); }
// Bit position of bit 4 of slot e of dword j inside the lane's high-plane word (5-bit).
W4_HD constexpr int hi_bit(int j, int e) {
  return (j == 0 ? 0 : j == 1 ? 2 : j == 2 ? 8 : 10) +
         (e == 0 ? 0 : e == 1 ? 16 : e == 2 ? 4 : e == 3 ? 20 : e == 4 ? 1 : e == 5 ? 17 : e == 6 ? 5 : 21);
}

}  // namespace w4layout
