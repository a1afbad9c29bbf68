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
constexpr int kGroup = 64;     // columns per scale/zero group

W4_HD constexpr int num_kblocks(int K) { return (K + kBlockK - 1) / kBlockK; }
W4_HD constexpr int block_bytes(int bits) { return bits == 5 ? 1280 : 1024; }

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
