// Host-side repacker: canonical groupwise weights -> the gfx950 packed layout.
//
// The packed layout (specified in include/w4gemm.h) puts each lane's codes in exactly the
// order the matrix-core A operand wants them, with the k order inside a 64-column group
// permuted so that one 32-bit word decodes into four fp16 pairs with a mask-and-or and the
// 4-bit low plane plus 1-bit high plane of 5-bit codes stay separate planes.  The freedom
// to permute k inside a group, provided the activations follow the same order, is the
// "Permuted k order" bullet of the ninfer-3080 performance notes ("What changed"); the
// split 5-bit form is the Q5 bullet of the same list.  Repacking is a pure permutation plus
// zero padding of a half-empty last k-block: bit-exact and deterministic.
#include <cstring>

#include "../../include/w4gemm.h"
#include "layout.h"

namespace {

using namespace w4layout;

bool shape_ok(int N, int K, int bits, int group) {
  return N > 0 && K > 0 && (N % kRowTile) == 0 && group_ok(group) && (K % k_multiple(group)) == 0 &&
         (bits == 4 || bits == 5);
}

inline int canonical_code(const uint8_t* lo, const uint8_t* hi, int K, int n, int k, int bits) {
  const uint8_t b = lo[(size_t)n * (K / 2) + (k >> 1)];
  int q = (k & 1) ? (b >> 4) : (b & 0xF);
  if (bits == 5) q |= ((hi[(size_t)n * (K / 8) + (k >> 3)] >> (k & 7)) & 1) << 4;
  return q;
}

// Repack source row tile `src_rt` of one canonical matrix into destination row tile `dst_rt`.
void repack_tile(const uint8_t* lo, const uint8_t* hi, const uint16_t* scales,
                 const uint16_t* zeros, int K, int bits, int group, int src_rt, int dst_rt,
                 uint8_t* w_out, uint16_t* s_out, uint16_t* z_out) {
  const int KB = num_kblocks(K);
  const int G = K / group;
  const size_t blk = block_bytes(bits);
  for (int kb = 0; kb < KB; ++kb) {
    uint8_t* block = w_out + ((size_t)dst_rt * KB + kb) * blk;
    for (int lane = 0; lane < 64; ++lane) {
      const int r = lane % 16, g = lane / 16;
      const int n = src_rt * kRowTile + r;
      uint32_t hiword = 0;
      for (int j = 0; j < 4; ++j) {
        uint32_t word = 0;
        for (int e = 0; e < 8; ++e) {
          const int k = slot_k(kb, g, j, e);
          const int q = (k < K) ? canonical_code(lo, hi, K, n, k, bits) : 0;
          word |= (uint32_t)(q & 0xF) << lo_bit(e);
          if (bits == 5) hiword |= (uint32_t)((q >> 4) & 1) << hi_bit(j, e);
        }
        std::memcpy(block + lane * 16 + j * 4, &word, 4);
      }
      if (bits == 5) std::memcpy(block + 64 * 16 + lane * 4, &hiword, 4);
    }
    // scale / zero-point words: word sz_word(group, r, g) of the block holds, in half h, the
    // group of the codes that row r's lane group g holds in its dwords 2h and 2h + 1 (columns
    // 64 h + 16 g .. 64 h + 16 g + 15 of the block)
    const int W = sz_words(group);
    for (int r = 0; r < kRowTile; ++r) {
      const int n = src_rt * kRowTile + r;
      for (int g = 0; g < 4; ++g) {
        for (int h = 0; h < 2; ++h) {
          const int grp = (kBlockK * kb + 64 * h + 16 * g) / group;
          const size_t o = (((size_t)dst_rt * KB + kb) * W + sz_word(group, r, g)) * 2 + h;
          s_out[o] = grp < G ? scales[(size_t)n * G + grp] : 0;
          z_out[o] = grp < G ? zeros[(size_t)n * G + grp] : 0;
        }
      }
    }
  }
}

}  // namespace

extern "C" size_t w4_packed_bytes(int N, int K, int bits, int group) {
  if (!shape_ok(N, K, bits, group)) return 0;
  return (size_t)(N / kRowTile) * num_kblocks(K) * block_bytes(bits);
}

extern "C" size_t w4_packed_sz_bytes(int N, int K, int group) {
  if (!shape_ok(N, K, 4, group)) return 0;
  return (size_t)(N / kRowTile) * num_kblocks(K) * sz_words(group) * 2 * sizeof(uint16_t);
}

extern "C" int w4_repack(const uint8_t* codes_lo, const uint8_t* codes_hi, const uint16_t* scales,
                         const uint16_t* zeros, int N, int K, int bits, int group, void* w_out,
                         uint16_t* scales_out, uint16_t* zeros_out) {
  if (bits != 4 && bits != 5) return W4_ERR_UNSUPPORTED;
  if (!group_ok(group)) return W4_ERR_UNSUPPORTED;
  if (!shape_ok(N, K, bits, group)) return W4_ERR_INVALID_ARG;
  if (!codes_lo || !scales || !zeros || !w_out || !scales_out || !zeros_out)
    return W4_ERR_INVALID_ARG;
  if ((bits == 5) != (codes_hi != nullptr)) return W4_ERR_INVALID_ARG;
  for (int rt = 0; rt < N / kRowTile; ++rt)
    repack_tile(codes_lo, codes_hi, scales, zeros, K, bits, group, rt, rt, (uint8_t*)w_out,
                scales_out, zeros_out);
  return W4_OK;
}

extern "C" int w4_repack_pair(const uint8_t* gate_lo, const uint8_t* gate_hi,
                              const uint16_t* gate_scales, const uint16_t* gate_zeros,
                              const uint8_t* up_lo, const uint8_t* up_hi,
                              const uint16_t* up_scales, const uint16_t* up_zeros, int N, int K,
                              int bits, int group, void* w_pair_out, uint16_t* scales_pair_out,
                              uint16_t* zeros_pair_out) {
  if (bits != 4 && bits != 5) return W4_ERR_UNSUPPORTED;
  if (!group_ok(group)) return W4_ERR_UNSUPPORTED;
  if (!shape_ok(N, K, bits, group)) return W4_ERR_INVALID_ARG;
  if (!gate_lo || !gate_scales || !gate_zeros || !up_lo || !up_scales || !up_zeros ||
      !w_pair_out || !scales_pair_out || !zeros_pair_out)
    return W4_ERR_INVALID_ARG;
  if ((bits == 5) != (gate_hi != nullptr) || (bits == 5) != (up_hi != nullptr))
    return W4_ERR_INVALID_ARG;
  for (int rt = 0; rt < N / kRowTile; ++rt) {
    repack_tile(gate_lo, gate_hi, gate_scales, gate_zeros, K, bits, group, rt, 2 * rt,
                (uint8_t*)w_pair_out, scales_pair_out, zeros_pair_out);
    repack_tile(up_lo, up_hi, up_scales, up_zeros, K, bits, group, rt, 2 * rt + 1,
                (uint8_t*)w_pair_out, scales_pair_out, zeros_pair_out);
  }
  return W4_OK;
}
