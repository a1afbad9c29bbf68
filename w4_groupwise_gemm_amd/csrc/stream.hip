// Streaming path for small and mid token counts: the GEMV route (exact T = 1..4, packed-fp16
// dot products) and the matrix-core routes for T <= 16, <= 32 and <= 64 (16-token steps).
//
// Prior art: the SIMT split GEMVs and the Q4/Q5 small-T MMA kernels of the ninfer-3080
// performance notes ("Why the round cost too much"; "What changed": permuted k order; "What
// is left at C1": at one stream the kernels are a streaming problem, ramp-up and drain).
//
// gfx950 design.  At these widths the kernel is an HBM stream with a dequantisation tax, so
// everything is arranged around keeping enough 16-byte code loads in flight and keeping the
// vector ALU work per packed word minimal:
//  * a workgroup owns RT 16-row tiles; its NW waves split K, wave w taking k-blocks w, w + NW,
//    w + 2 NW, ... (at any moment the workgroup streams NW adjacent blocks of a tile), so each
//    code byte is loaded exactly once, into the lane that feeds it to the math;
//  * each wave keeps a ring of D k-blocks of loads in flight ahead of the math (with one row
//    tile, all of its blocks: the stream never waits for the math); code loads are
//    non-temporal (each byte is read once per call);
//  * the wave's activation slice (the token rows of its k-blocks) is loaded first and parked
//    in a wave-private LDS region, so activation reads never wait behind code loads in the
//    in-order load counter and no barrier is needed inside the loop: for K <= 5120, 4, 8 or 16
//    rows straight from memory (direct-to-LDS loads, no registers), the 8- and 16-row ones with
//    1 to 3 row tiles per workgroup chosen for an even spread over the compute units, since
//    the slice then allows only one or two workgroups per compute unit; for longer K, 4 rows
//    through registers (T <= 4), or the 16-token activation fragments ride in the same ring as
//    the codes;
//  * for 17-64 tokens (K <= 5120) a whole slice no longer fits: each wave keeps a ring of
//    32-row (two slots) or 64-row (one slot) activation tiles, refilled from memory as blocks
//    are consumed, and feeds every dequantised weight fragment to 2 or 4 16-token steps; the
//    waits count the loads issued after each tile, so scheduling barriers keep every tile
//    load of the prologue ahead of the code loads;
//  * the dequantisation is 13 vector ops per packed word when the zero-points of a block are
//    integers (checked exactly, wave-uniformly, per block): mask-or the nibbles into the
//    mantissa of fp16 1024 (one v_and_or_b32 per pair), subtract 1024 + z (or fold 1/16 and
//    64 + z into one packed fma for the high-nibble pairs) and multiply by the scale;
//    fractional zero-points take the general 17-op form;
//  * token rows beyond T are clamped to row T-1 instead of masked: those output columns are
//    never stored, so the loads need no exec masking;
//  * the NW partial sums are combined in LDS in a fixed order (bitwise deterministic).
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace w4 {
namespace {

using namespace w4dev;
using w4layout::block_bytes;

enum { MODE_MFMA = 0, MODE_DOT2 = 1 };

// fp16 weights (q - z) * s of dword J as four pairs.  FAST: z is an integer (1024 + z and
// 64 + z exact in fp16), b0 = -(1024 + z), b1 = -(64 + z).  Otherwise q is made exact first.
template <int BITS, int J, bool FAST>
__device__ __forceinline__ void weights(uint32_t w, uint32_t hiw, uint32_t magic, f16x2 z2, f16x2 b0,
                                        f16x2 b1, f16x2 s2, f16x2 out[4]) {
  uint32_t u[4];
  wbiased<BITS, J>(w, hiw, magic, u);
  const f16x2 c16th = {(f16)0.0625f, (f16)0.0625f};
  if constexpr (FAST) {
    out[0] = (as_h2(u[0]) + b0) * s2;
    out[1] = (as_h2(u[1]) * c16th + b1) * s2;
    out[2] = (as_h2(u[2]) + b0) * s2;
    out[3] = (as_h2(u[3]) * c16th + b1) * s2;
  } else {
    const f16x2 c1024 = {(f16)1024.0f, (f16)1024.0f}, c64 = {(f16)64.0f, (f16)64.0f};
    out[0] = ((as_h2(u[0]) - c1024) - z2) * s2;
    out[1] = ((as_h2(u[1]) * c16th - c64) - z2) * s2;
    out[2] = ((as_h2(u[2]) - c1024) - z2) * s2;
    out[3] = ((as_h2(u[3]) * c16th - c64) - z2) * s2;
  }
}

// The same for an n that is a constant once the caller's loop is unrolled.
template <int N = 0>
__device__ __forceinline__ void wait_vmcnt_folded(int n) {
  if constexpr (N < 63) {
    if (n == N) {
      wait_vmcnt<N>();
      return;
    }
    wait_vmcnt_folded<N + 1>(n);
  } else {
    wait_vmcnt<63>();
  }
}

template <int BITS, int RT, int KPW, int XL>
struct Ring {
  u32x4 cw[KPW][RT];
  uint32_t hw[KPW][RT], sp[KPW][RT], zp[KPW][RT];
  u32x4 xb[XL ? 1 : KPW][4];
};

// Whether the activation slice goes straight from memory to LDS (direct-to-LDS loads, 16-byte
// chunks XOR-swizzled by token row): always for 8 and 16 rows, and for 4 rows when a wave's
// blocks form one chunk of at most five (K <= 5120).  Longer K keeps the 4-row slice in padded
// rows loaded through registers, chunk by chunk.  (Decode 12288 x 5120, T = 1 / 2 / 4: 8.55 /
// 8.61 / 9.16 us direct, 8.71 / 8.90 / 9.48 through registers.)
template <int XL, int KPW, bool LOOP>
constexpr bool slice_dma() {
  return XL == 8 || XL == 16 || (XL == 4 && KPW <= 5 && !LOOP);
}

// XL: token rows of the activation slice held in LDS (0: fragments in the ring instead; 4, 8
// or 16; 32: a two-block ring of 32-row activation tiles, refilled as the blocks are consumed,
// and two 16-token matrix-core steps per weight fragment; 64: one 64-row tile slot, refilled
// with the next block's tile as soon as the current one has been read, and four steps).
// xdim: the slice's k-blocks (direct-to-LDS slices), or fp16 elements per padded row (4 rows
// through registers).
// HB: K is not a multiple of 128, so the last k-block holds one group only (without it the
// per-block test for that case, and its branches, compile away).
// bx: the workgroup's index among those of this matrix (its row tiles are bx RT ..).
// ring0 / ring1 (two-slot 32-row ring only): slot 0 and slot 1 of every wave, one array each.
// A direct-to-LDS refill is a write the compiler cannot place within an array, so before any
// LDS read it waits for the newest refill into the same array; with the two slots in distinct
// arrays, reading slot (i + 1) % 2 no longer waits for the refill of slot i % 2 (and for every
// load issued before it).
template <int BITS, int MODE, int RT, int NW, int KPW, int D, int XL, int EPI, bool LOOP, bool HB>
__device__ __forceinline__ void stream_body(const KArgs& a, int xdim, int bx, char* ring0, char* ring1) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int BLK = block_bytes(BITS);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int szl = sz_lane_word(a, r, g);  // the lane's scale / zero-point word in a block
  const int ntiles = a.rows / 16;
  const int tile0 = bx * RT;
  // local block index c of this wave is k-block wave + NW * c; nbw of them
  const int nbw = wave < a.KB ? (a.KB - wave + NW - 1) / NW : 0;
  const int T = a.T;
  const int tr = min(r, T - 1);
  const uint32_t magic = vgpr_const(0x64006400u);
  // Wave-private activation slice.  Direct-to-LDS (4, 8 or 16 rows): XL x 256 B per k-block,
  // block after block, 16-byte chunk j of row t stored at chunk j ^ t (no padding: at K = 5120
  // two 8-row or one 16-row workgroup slice fill the LDS exactly).  4 rows through registers:
  // row t holds the chunk's blocks back to back, rows xdim elements apart (16 bytes of padding:
  // the rows a fragment read touches hit distinct banks).
  // 32 / 64 rows: two / one slots of XL rows x 256 B (block i in slot i % 2 / slot 0), chunk j
  // of row t at j ^ (t % 16).
  constexpr bool RING = XL >= 32;
  constexpr bool XDMA = slice_dma<XL, KPW, LOOP>();  // direct-to-LDS slice
  constexpr bool XREG = XL == 4 && !XDMA;            // 4-row slice through registers
  // Token row of this lane's B column in a direct-to-LDS slice or ring tile: row r itself (mod
  // the tile's rows), not the clamped T - 1.  Rows at or beyond T hold zeros (the loads past the
  // end of X read zero) and feed output columns that are never stored; keeping the 16 rows of a
  // read distinct keeps it free of bank conflicts under the XOR swizzle (with the clamp, T = 4
  // and T = 8 cost about 80 conflict cycles per wave).
  const int tl = XDMA || RING ? (r & (XL - 1)) : tr;
  constexpr int TH = RING ? XL / 16 : 1;  // 16-token groups per weight fragment
  constexpr int NSLOT = XL == 32 ? 2 : 1;
  constexpr int XBLK = XL * 256;
  char* const xs = NSLOT == 2 ? nullptr
                  : smem + (size_t)wave * (RING ? NSLOT * XBLK : XDMA ? xdim * XBLK : XL * xdim * 2);
  // slot of local block i (i is a constant once the block loop is unrolled)
  auto xslot = [&](int i) -> char* {
    if constexpr (NSLOT == 2)
      return (i % 2 ? ring1 : ring0) + (size_t)wave * XBLK;
    else
      return xs;
  };
  // 16-byte chunk c (0..15) of token row t of local block i
  auto xchunk = [&](int i, int t, int c) -> const char* {
    if constexpr (RING)
      return xslot(i) + t * 256 + ((c ^ (t & 15)) << 4);
    else if constexpr (XDMA)
      return xs + i * XBLK + t * 256 + ((c ^ t) << 4);
    else
      return xs + (t * xdim + i * 128 + c * 8) * 2;
  };
  const auto xres = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(a.x), (short)0,
                                                      (int)((size_t)a.T * a.K * 2), 0x00020000);
  // acc: tokens 0..15; accx[q - 1]: tokens 16 q .. 16 q + 15
  f32x4 acc[RT], accx[TH > 1 ? TH - 1 : 1][RT];
  float accd[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q + 1 < TH; ++q) accx[q][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) accd[rt][t] = 0.f;
  }

  Ring<BITS, RT, KPW, XL> R;
  // Without LOOP the launcher guarantees at most one chunk per wave (nbw <= KPW): a runtime
  // loop around the unrolled ring costs about a third more registers.  A wave without blocks
  // (K shorter than NW k-blocks) skips the body entirely.
  for (int cb = 0; LOOP ? cb < nbw : (cb == 0 && cb < nbw); cb += KPW) {
    const int nb = min(KPW, nbw - cb);

    // activation slice of this chunk, loaded before any code of the chunk.  Direct-to-LDS: one
    // instruction per 4 token rows of a block (lane L: row 4h + L/16, stored chunk L%16 =
    // source chunk (L%16) ^ row); rows at or beyond T lie past the end of the range-checked
    // buffer and read as zero.  Through registers: T <= 4 rows of nb k-blocks.
    constexpr int XCH = (KPW * 16 + 63) / 64;  // 16-byte chunks per lane per token row
    u32x4 xr[XREG ? 4 : 1][XREG ? XCH : 1];
    if constexpr (XREG) {
      const int cpt = nb * 16;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < T) {
#pragma unroll
          for (int i = 0; i < XCH; ++i) {
            const int c = min(lane + 64 * i, cpt - 1);
            const int kk = min((wave + NW * (cb + (c >> 4))) * 128 + (c & 15) * 8, a.K - 8);
            xr[t][i] = *reinterpret_cast<const u32x4*>(a.x + (size_t)t * a.K + kk);
          }
        }
      }
    } else if constexpr (XDMA) {
      static_assert(!LOOP, "direct-to-LDS slices hold one chunk");
#pragma unroll
      for (int ib = 0; ib < KPW; ++ib) {
        // (KPW == nb here: the launcher picks the chunk size equal to the wave's block count)
        const int kb = wave + NW * ib;
#pragma unroll
        for (int h = 0; h < XL / 4; ++h) {
          const int t = 4 * h + (lane >> 4);
          const int off = (t * a.K + kb * 128 + (((lane & 15) ^ t) << 3)) * 2;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (__attribute__((address_space(3))) void*)(xs + ib * XBLK + h * 1024),
                                                   16, off, 0, 0, 0);
        }
      }
      // the waits below count loads issued after the slice: keep every slice load ahead of the
      // code loads (the scheduler may otherwise interleave them)
      __builtin_amdgcn_sched_barrier(0);
    }

    // 32 / 64 rows: the tile of local block i into its ring slot (XL / 4 direct-to-LDS
    // instructions of 4 token rows each, laid out as above).
    auto xload = [&](int i) {
      const int kb = wave + NW * (cb + min(i, nb - 1));
#pragma unroll
      for (int h = 0; h < XL / 4; ++h) {
        const int t = 4 * h + (lane >> 4);
        const int off = (t * a.K + kb * 128 + (((lane & 15) ^ (t & 15)) << 3)) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (__attribute__((address_space(3))) void*)(xslot(i) + h * 1024),
                                                 16, off, 0, 0, 0);
      }
    };
    if constexpr (RING) {
      static_assert(!LOOP, "the activation ring holds one chunk");
      xload(0);
      if constexpr (NSLOT == 2) xload(1);
      __builtin_amdgcn_sched_barrier(0);  // (as for the slice: the waits count loads after these)
    }

    // Loads of local block i.  The first D blocks are issued unconditionally (a wave with
    // fewer blocks re-reads its last one), so that the compiler counts the loads in flight
    // exactly and waits for each block alone rather than for the whole ring.
    auto issue = [&](int i) {
      const int kb = wave + NW * (cb + min(i, nb - 1));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int tile = min(tile0 + rt, ntiles - 1);
        const size_t bi = (size_t)tile * a.KB + kb;
        R.cw[i][rt] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.w + bi * BLK + lane * 16));
        if constexpr (BITS == 5)
          R.hw[i][rt] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a.w + bi * BLK + 1024 + lane * 4));
        else
          R.hw[i][rt] = 0;
        R.sp[i][rt] = a.sc[bi * a.szw + szl];
        R.zp[i][rt] = a.zr[bi * a.szw + szl];
      }
      if constexpr (XL == 0) {
        const bool half_block = HB && (kb * 128 + 64 >= a.K);
        const _Float16* xrow = a.x + (size_t)tr * a.K + kb * 128 + 16 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          R.xb[i][j] = (half_block && j >= 2)
                           ? u32x4{0u, 0u, 0u, 0u}
                           : *reinterpret_cast<const u32x4*>(xrow + 64 * (j >> 1) + 8 * (j & 1));
      }
    };
    static_assert(D <= KPW, "ring deeper than the chunk");
#pragma unroll
    for (int i = 0; i < D; ++i) issue(i);

    if constexpr (XREG) {
      const int cpt = nb * 16;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < T) {
#pragma unroll
          for (int i = 0; i < XCH; ++i) {
            const int c = lane + 64 * i;
            if (c < cpt) *reinterpret_cast<u32x4*>(xs + (t * xdim + c * 8) * 2) = xr[t][i];
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else if constexpr (XDMA) {
      // the slice has landed once at most the ring prologue's loads are outstanding
      wait_vmcnt<D * RT * (BITS == 5 ? 4 : 3)>();
    }

#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      // (ring modes issue every slot, re-reading a wave's last block past its end, so that the
      // tile waits below can count the loads issued after each tile)
      // (the two-slot ring issues its code loads with its tile refills, below)
      if (NSLOT != 2 && i + D < KPW && (RING || i + D < nb)) issue(i + D);
      if (i < nb) {
        const int kb = wave + NW * (cb + i);
        const bool half_block = HB && (kb * 128 + 64 >= a.K);
        // activation fragments of the block's four 32-k steps, read before the dequantisation
        // so that the LDS latency hides behind it (a half-empty last block skips steps 2, 3)
        f16x8 Bf[4], Bx[TH > 1 ? TH - 1 : 1][4];
        if constexpr (RING) {
          // The ring tile of block i has landed once at most the loads issued after it are
          // outstanding.  CPB: code loads per block.
          //  * Two slots: tiles 0 and 1, code blocks 0 .. D-1 (D = 2); after block i's math the
          //    refill of tile i + 2, then code block i + 2.  A code block thus follows every
          //    tile load issued before its own block's tile, so the compiler's wait for its
          //    registers (which counts only register loads) waits for at most the next block's
          //    tile besides, never for later code blocks.
          //  * One slot: tile 0, code blocks 0 .. D-1; then code block i + D at the top of
          //    block i, and the refill of tile i + 1 right after block i's tile has been read.
          constexpr int CPB = RT * (BITS == 5 ? 4 : 3);
          int n;
          if constexpr (NSLOT == 2)
            n = i == 0 ? 8 + D * CPB
              : i == 1 ? D * CPB + (2 < KPW ? 8 + CPB : 0)
              : CPB + (i + 1 < KPW ? 8 + CPB : 0);
          else
            n = i == 0 ? CPB * (D + (D < KPW ? 1 : 0)) : CPB * (i + D < KPW);
          wait_vmcnt_folded(n);
        }
        if constexpr (MODE == MODE_MFMA) {
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            if constexpr (XL > 0)
              Bf[J] = *reinterpret_cast<const f16x8*>(xchunk(i, tl, 8 * (J >> 1) + 2 * g + (J & 1)));
            else
              Bf[J] = __builtin_bit_cast(f16x8, R.xb[i][J]);
#pragma unroll
            for (int q = 0; q + 1 < TH; ++q)
              Bx[q][J] = *reinterpret_cast<const f16x8*>(xchunk(i, (16 * (q + 1) + r) & (XL - 1), 8 * (J >> 1) + 2 * g + (J & 1)));
          }
        }
        if constexpr (XL == 64) {
          if (i + 1 < KPW) {
            // the tile has been read: refill the slot with the next block's tile under this
            // block's math
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt 0 (vmcnt, expcnt: no wait)
            xload(i + 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          // exact wave-uniform test: are both zero-points of this block integers?
          const f16x2 z2p = as_h2(R.zp[i][rt]);
          const f16x2 c1024 = {(f16)1024.0f, (f16)1024.0f}, c64 = {(f16)64.0f, (f16)64.0f};
          const f16x2 nb0 = -(z2p + c1024);
          const bool exact = __builtin_bit_cast(uint32_t, (-nb0) - c1024) == R.zp[i][rt];
          const bool fast = __ballot(exact) == ~0ull;
          const f16x2 nb1 = -(z2p + c64);
          // fp16 weights of dword J (8 k slots of the lane's row) as four pairs
          auto wts = [&](auto jc, bool is_fast, f16x2 (&wv)[4]) {
            constexpr int J = decltype(jc)::value;
            const f16x2 s2 = splat<(J >> 1)>(R.sp[i][rt]);
            if (is_fast)
              weights<BITS, J, true>(R.cw[i][rt][J], R.hw[i][rt], magic, f16x2{},
                                     splat<(J >> 1)>(__builtin_bit_cast(uint32_t, nb0)),
                                     splat<(J >> 1)>(__builtin_bit_cast(uint32_t, nb1)), s2, wv);
            else
              weights<BITS, J, false>(R.cw[i][rt][J], R.hw[i][rt], magic,
                                      splat<(J >> 1)>(R.zp[i][rt]), f16x2{}, f16x2{}, s2, wv);
          };
          if constexpr (MODE == MODE_MFMA) {
            // all four A fragments first (one uniform branch per block), then the four steps
            f16x8 A[4];
            auto all_a = [&](bool is_fast) {
              f16x2 wv[4];
              wts(std::integral_constant<int, 0>{}, is_fast, wv);
              A[0] = cat8(wv[0], wv[1], wv[2], wv[3]);
              wts(std::integral_constant<int, 1>{}, is_fast, wv);
              A[1] = cat8(wv[0], wv[1], wv[2], wv[3]);
              if (!half_block) {
                wts(std::integral_constant<int, 2>{}, is_fast, wv);
                A[2] = cat8(wv[0], wv[1], wv[2], wv[3]);
                wts(std::integral_constant<int, 3>{}, is_fast, wv);
                A[3] = cat8(wv[0], wv[1], wv[2], wv[3]);
              }
            };
            if (fast)
              all_a(true);
            else
              all_a(false);
            auto steps = [&](int J) {
              acc[rt] = mfma16(A[J], Bf[J], acc[rt]);
#pragma unroll
              for (int q = 0; q + 1 < TH; ++q) accx[q][rt] = mfma16(A[J], Bx[q][J], accx[q][rt]);
            };
            steps(0);
            steps(1);
            if (!half_block) {
              steps(2);
              steps(3);
            }
          } else {
            auto dot_j = [&](auto jc) {
              constexpr int J = decltype(jc)::value;
              if (half_block && J >= 2) return;
              f16x2 wv[4];
              wts(jc, fast, wv);
              const int c = 8 * (J >> 1) + 2 * g + (J & 1);
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                if (t < T) {
                  const u32x4 xv = *reinterpret_cast<const u32x4*>(xchunk(i, t, c));
                  float v = accd[rt][t];
#pragma unroll
                  for (int p = 0; p < 4; ++p) v = __builtin_amdgcn_fdot2(wv[p], as_h2(xv[p]), v, false);
                  accd[rt][t] = v;
                }
              }
            };
            dot_j(std::integral_constant<int, 0>{});
            dot_j(std::integral_constant<int, 1>{});
            dot_j(std::integral_constant<int, 2>{});
            dot_j(std::integral_constant<int, 3>{});
          }
        }
      }
      if constexpr (XL == 32) {
        if (i + 2 < KPW) {
          // this wave's reads of slot i % 2 are complete: refill it with block i + 2's tile,
          // then issue block i + 2's codes
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt 0 (vmcnt, expcnt: no wait)
          xload(i + 2);
          __builtin_amdgcn_sched_barrier(0);
          issue(i + 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // ---- fixed-order combination of the NW partial sums, then the epilogue
  __syncthreads();
  if constexpr (MODE == MODE_MFMA) {
    // red[w][h][rt][lane]: wave w's partial sums of token half h, row tile rt (the two-slot
    // ring's first array holds them there: NW x 2 x RT KB within its NW x 8 KB)
    f32x4* red = reinterpret_cast<f32x4*>(NSLOT == 2 ? ring0 : smem);
    static_assert(NSLOT != 2 || TH * RT * 1024 <= XBLK, "reduction fits the ring's first array");
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      red[((wave * TH + 0) * RT + rt) * 64 + lane] = acc[rt];
#pragma unroll
      for (int q = 0; q + 1 < TH; ++q) red[((wave * TH + q + 1) * RT + rt) * 64 + lane] = accx[q][rt];
    }
    __syncthreads();
    auto sum = [&](int h, int rt, int l) {
      f32x4 v = red[(h * RT + rt) * 64 + l];
      for (int w = 1; w < NW; ++w) v = v + red[((w * TH + h) * RT + rt) * 64 + l];
      return v;
    };
    constexpr int ITEMS = TH * (EPI == EPI_SWIGLU ? RT / 2 : RT) * 64;
    for (int it = threadIdx.x; it < ITEMS; it += NW * 64) {
      const int l = it & 63, hp = it >> 6;
      const int h = hp % TH, p = hp / TH;
      const int t = 16 * h + (l & 15);
      if (t >= T) continue;
      if constexpr (EPI == EPI_SWIGLU) {
        const int gtile = tile0 + 2 * p;
        if (gtile >= ntiles) continue;
        store_quad<EPI>(a, t, (gtile >> 1) * 16 + 4 * (l >> 4), sum(h, 2 * p, l),
                        sum(h, 2 * p + 1, l));
      } else {
        const int tile = tile0 + p;
        if (tile >= ntiles) continue;
        store_quad<EPI>(a, t, tile * 16 + 4 * (l >> 4), sum(h, p, l), f32x4{});
      }
    }
  } else {
    float* red = reinterpret_cast<float*>(smem);  // [NW][RT][4][16]
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float v = accd[rt][t];
        v = v + __shfl_xor(v, 16);
        v = v + __shfl_xor(v, 32);
        if (lane < 16) red[((wave * RT + rt) * 4 + t) * 16 + lane] = v;
      }
    __syncthreads();
    constexpr int ITEMS = (EPI == EPI_SWIGLU ? RT / 2 : RT) * 64;
    for (int it = threadIdx.x; it < ITEMS; it += NW * 64) {
      const int row = it & 15, t = (it >> 4) & 3, p = it >> 6;
      if (t >= T) continue;
      if constexpr (EPI == EPI_SWIGLU) {
        const int gtile = tile0 + 2 * p;
        if (gtile >= ntiles) continue;
        float gv = red[((2 * p) * 4 + t) * 16 + row], uv = red[((2 * p + 1) * 4 + t) * 16 + row];
        for (int w = 1; w < NW; ++w) {
          gv += red[((w * RT + 2 * p) * 4 + t) * 16 + row];
          uv += red[((w * RT + 2 * p + 1) * 4 + t) * 16 + row];
        }
        store_one<EPI>(a, t, (gtile >> 1) * 16 + row, gv, uv);
      } else {
        const int tile = tile0 + p;
        if (tile >= ntiles) continue;
        float v = red[(p * 4 + t) * 16 + row];
        for (int w = 1; w < NW; ++w) v += red[((w * RT + p) * 4 + t) * 16 + row];
        store_one<EPI>(a, t, tile * 16 + row, v, 0.f);
      }
    }
  }
}

template <int BITS, int MODE, int RT, int NW, int KPW, int D, int XL, int EPI, bool LOOP, bool HB>
__global__ __launch_bounds__(NW * 64) void stream_kernel(KArgs a, int xdim) {
  if constexpr (XL == 32) {
    __shared__ __attribute__((aligned(16))) char ring0[NW * 32 * 256], ring1[NW * 32 * 256];
    stream_body<BITS, MODE, RT, NW, KPW, D, XL, EPI, LOOP, HB>(a, xdim, blockIdx.x, ring0, ring1);
  } else {
    stream_body<BITS, MODE, RT, NW, KPW, D, XL, EPI, LOOP, HB>(a, xdim, blockIdx.x, nullptr, nullptr);
  }
}

// Grouped launch: several matrices (4- or 5-bit) that share one activation, each with its own
// output; workgroups [end[p-1], end[p]) run matrix p.
struct GArgs {
  KArgs a[kMaxParents];
  int bits[kMaxParents];
  int end[kMaxParents];  // exclusive prefix sums of the matrices' workgroup counts
  int n;
};

template <int MODE, int RT, int NW, int KPW, int D, int XL, int EPI, bool LOOP, bool HB>
__global__ __launch_bounds__(NW * 64) void stream_grouped_kernel(GArgs g, int xdim) {
  int p = 0;
  while (p + 1 < g.n && (int)blockIdx.x >= g.end[p]) ++p;
  const int bx = blockIdx.x - (p > 0 ? g.end[p - 1] : 0);
  if constexpr (XL == 32) {
    __shared__ __attribute__((aligned(16))) char ring0[NW * 32 * 256], ring1[NW * 32 * 256];
    if (g.bits[p] == 5)
      stream_body<5, MODE, RT, NW, KPW, D, XL, EPI, LOOP, HB>(g.a[p], xdim, bx, ring0, ring1);
    else
      stream_body<4, MODE, RT, NW, KPW, D, XL, EPI, LOOP, HB>(g.a[p], xdim, bx, ring0, ring1);
  } else {
    if (g.bits[p] == 5)
      stream_body<5, MODE, RT, NW, KPW, D, XL, EPI, LOOP, HB>(g.a[p], xdim, bx, nullptr, nullptr);
    else
      stream_body<4, MODE, RT, NW, KPW, D, XL, EPI, LOOP, HB>(g.a[p], xdim, bx, nullptr, nullptr);
  }
}

constexpr int kNW = 8;  // waves per workgroup (K split)
// Ring depth (k-blocks of loads in flight ahead of the math).  One row tile with the
// activation slice in LDS: 5, every block of a 5120-column wave in flight at once (decode
// 12288 x 5120, T = 1: 11.1 us with 3, 10.6 us with 5).  Activation fragments in the ring
// (T > 4): 3, since each stage then costs 16 more registers.  Two row tiles with a 4-row
// slice: 2, where the smaller register footprint buys more resident waves (SwiGLU pair, 34816
// packed rows, T = 1: 26.5 us against 30.0 us with 3).  Two row tiles with an 8-row slice: the
// 80 KB slice already limits a compute unit to two workgroups, so all 5 blocks.  Never deeper
// than the chunk.  Three row tiles with an 8- or 16-row slice: likewise 5.  Six row tiles (the
// SwiGLU pair with a 16-row slice): 2, within the registers of the one workgroup per compute
// unit that the slice allows.
// Row tiles per workgroup where a launch holds about one round of workgroups (the 8- and
// 16-row slices and the 32- / 64-row rings, which allow two or one workgroups per compute unit).
// Workgroups are taken round-robin over the 256 compute units in launch order; a compute unit's
// cost is the code bits of the row tiles it runs, plus a start-up cost per workgroup (its
// activation slice or ring prologue and its final reduction): half a 4-bit tile with a slice,
// a tile and a half with a ring, which also allows only one workgroup per compute unit at a
// time.  The count (1 .. max_rt) with the smallest largest cost wins; ties go to more tiles
// (fewer workgroups).  Measured at K = 5120 (us; one, two, three row tiles per workgroup):
//   4-bit  4096 rows: T = 8   5.4 /  7.1 /  8.4    T = 32  7.6 /  9.0 / 10.9   (one wins)
//   4-bit  7168 rows: T = 16 10.0 /  8.3 /  9.7    T = 32 13.1 / 10.2 / 11.6   (two)
//   4-bit 11264 rows: T = 16 14.5 / 14.4 / 11.1    T = 64 27.4 / 24.4 / 18.1   (three)
//   5-bit 12288 rows: T = 16 17.3 / 17.1 / 14.1    T = 32 21.7 / 20.9 / 16.8   (three)
//   5-bit 12288 rows, T = 64 (at most two: see pick_rt): 29.5 / 27.4                (two)
// and for the groups of the grouped launch (4-bit 4096 + 5-bit 12288 rows, T = 8: 16.0 / 15.1 /
// 20.1 us; two).
struct TileGroup {
  int tiles;  // 16-row tiles of one matrix
  int bits;   // its code width
};

inline int launch_cost(const TileGroup* m, int n, int rt, int start) {
  constexpr int kCUs = 256;
  if (n == 1) {  // one matrix: the busiest compute unit runs ceil(workgroups / 256) of them
    const int nwg = (m[0].tiles + rt - 1) / rt;
    return (rt * m[0].bits + start) * ((nwg + kCUs - 1) / kCUs);
  }
  int first = 0;  // index of the matrix's first workgroup in the launch
  int worst = 0;
  int cost[kCUs] = {};
  for (int p = 0; p < n; ++p) {
    const int nwg = (m[p].tiles + rt - 1) / rt;
    const int w = rt * m[p].bits + start;
    // workgroups first .. first + nwg - 1 land on compute units (first + i) % 256
    const int full = nwg / kCUs, rest = nwg % kCUs;
    for (int c = 0; c < kCUs; ++c) {
      const int extra = ((c - first % kCUs + kCUs) % kCUs) < rest ? 1 : 0;
      cost[c] += w * (full + extra);
    }
    first += nwg;
  }
  for (int c = 0; c < kCUs; ++c) worst = cost[c] > worst ? cost[c] : worst;
  return worst;
}

// start: the start-up cost per workgroup, in bits of one 16-row tile (2 with an activation
// slice, 6 with a ring)
inline int tiles_per_workgroup(const TileGroup* m, int n, int max_rt, int start) {
  int best = max_rt, best_cost = launch_cost(m, n, max_rt, start);
  for (int rt = max_rt - 1; rt >= 1; --rt) {
    const int c = launch_cost(m, n, rt, start);
    if (c < best_cost) best = rt, best_cost = c;
  }
  return best;
}

inline int tiles_per_workgroup(int ntiles, int bits, int max_rt, int start) {
  const TileGroup m{ntiles, bits};
  return tiles_per_workgroup(&m, 1, max_rt, start);
}

template <int RT, int XL, int KPW>
constexpr int ring_depth() {
  constexpr int d = XL == 32 ? 2 : XL >= 32 ? 5 : XL >= 8 ? (RT >= 6 ? 2 : 5) : RT >= 2 ? 2 : (XL ? 5 : 3);
  return d < KPW ? d : KPW;
}

// Dynamic LDS of one workgroup: the activation slice or ring (nbc blocks per chunk; xdim as
// passed to the kernel), or the final reduction of the NW partial sums if that is larger.
template <int MODE, int RT, int XL, bool DMA>
size_t stream_lds(int nbc, int xdim) {
  if constexpr (XL == 32) return 0;  // the two-slot ring and its reduction live in static arrays
  const size_t x = XL == 32 ? (size_t)kNW * 2 * 32 * 256
                 : XL == 64 ? (size_t)kNW * 64 * 256
                 : DMA ? (size_t)kNW * nbc * XL * 256 : XL == 4 ? (size_t)kNW * 4 * xdim * 2 : 0;
  const size_t red = MODE == MODE_MFMA ? (size_t)kNW * RT * (XL >= 32 ? XL / 16 : 1) * 64 * 16
                                       : (size_t)kNW * RT * 64 * 4;
  return red > x ? red : x;
}

template <int BITS, int MODE, int RT, int XL, int EPI, int KPW, bool LOOP>
hipError_t run_k(const KArgs& a, hipStream_t stream) {
  const int ntiles = a.rows / 16;
  const int nbw = (a.KB + kNW - 1) / kNW;
  const int nbc = nbw < KPW ? nbw : KPW;  // blocks per chunk
  constexpr bool DMA = slice_dma<XL, KPW, LOOP>();
  const int xdim = DMA ? nbc : nbc * 128 + 8;
  const size_t lds = stream_lds<MODE, RT, XL, DMA>(nbc, xdim);
  constexpr int D = ring_depth<RT, XL, KPW>();
  const dim3 grid((ntiles + RT - 1) / RT), block(kNW * 64);
  if (a.K % 128)
    return launch_kernel(&stream_kernel<BITS, MODE, RT, kNW, KPW, D, XL, EPI, LOOP, true>, grid, block,
                         lds, stream, a, xdim);
  return launch_kernel(&stream_kernel<BITS, MODE, RT, kNW, KPW, D, XL, EPI, LOOP, false>, grid, block,
                       lds, stream, a, xdim);
}

// k-blocks per wave: one unrolled chunk (exactly the wave's block count up to 5, so that no
// ring slot is a re-read), up to 8 blocks with a 4-row activation slice and up to 16 with
// fragments in the ring; a chunk loop beyond.  A 4-row slice of more than 8 blocks per wave
// would take more than 80 KB of LDS (96 KB at K = 12288), one workgroup per compute unit, and
// a 5120-row launch (320 workgroups) would then run in two rounds: 19.8 us at T = 1 with 5-bit
// codes, against 11.1 at K = 8192 and 23.0 at K = 17408 (8-block chunks).
template <int BITS, int MODE, int RT, int XL, int EPI>
hipError_t run(const KArgs& a, hipStream_t stream) {
  const int nbw = (a.KB + kNW - 1) / kNW;
  if (nbw <= 1) return run_k<BITS, MODE, RT, XL, EPI, 1, false>(a, stream);
  if (nbw == 2) return run_k<BITS, MODE, RT, XL, EPI, 2, false>(a, stream);
  if (nbw == 3) return run_k<BITS, MODE, RT, XL, EPI, 3, false>(a, stream);
  if (nbw == 4) return run_k<BITS, MODE, RT, XL, EPI, 4, false>(a, stream);
  if (nbw == 5) return run_k<BITS, MODE, RT, XL, EPI, 5, false>(a, stream);
  if constexpr (XL >= 8) {
    return hipErrorInvalidValue;  // 8- and 16-row slices are picked for K <= 5120 only
  } else {
    if (nbw <= 8) return run_k<BITS, MODE, RT, XL, EPI, 8, false>(a, stream);
    if constexpr (XL == 0) {
      if (nbw <= 16) return run_k<BITS, MODE, RT, XL, EPI, 16, false>(a, stream);
    }
    return run_k<BITS, MODE, RT, XL, EPI, 8, true>(a, stream);
  }
}

template <int BITS, int MODE, int XL, int EPI>
hipError_t pick_rt(const KArgs& a, hipStream_t stream) {
  const int ntiles = a.rows / 16;
  if constexpr (EPI == EPI_SWIGLU) {
    // the gate / up tiles of one pair.  With a 16-row slice (one 160 KB workgroup per compute
    // unit) one or three pairs, by the balance rule with a start-up cost of a tile and a half
    // per workgroup: 17408-row pair, T = 16: 33.0 us with three against 35.4 with one; 8192
    // rows 17.0 against 16.1; 4096 rows (86 workgroups with three) 15.6 against 8.7.
    // Otherwise one pair (every other width and size measured best so, e.g. 17408 rows, T = 8:
    // 24.7 against 32.2 us with three).
    if constexpr (XL == 16) {
      const TileGroup m{ntiles, BITS};
      if (launch_cost(&m, 1, 2, 6) < launch_cost(&m, 1, 6, 6))
        return run<BITS, MODE, 2, XL, EPI>(a, stream);
      return run<BITS, MODE, 6, XL, EPI>(a, stream);
    } else {
      return run<BITS, MODE, 2, XL, EPI>(a, stream);
    }
  } else if constexpr (XL >= 8) {
    // an 8-row slice (80 KB at K = 5120) leaves room for two workgroups per compute unit, a
    // 16-row one or a 32- / 64-row ring for one, so the row tiles per workgroup decide how
    // evenly a launch spreads over the compute units (tiles_per_workgroup); three row tiles of
    // 5-bit codes with 64-token accumulators exceed the registers
    const int rt = tiles_per_workgroup(ntiles, BITS, XL == 64 && BITS == 5 ? 2 : 3, XL >= 32 ? 6 : 2);
    if (rt == 1) return run<BITS, MODE, 1, XL, EPI>(a, stream);
    if constexpr (!(XL == 64 && BITS == 5)) {
      if (rt == 3) return run<BITS, MODE, 3, XL, EPI>(a, stream);
    }
    return run<BITS, MODE, 2, XL, EPI>(a, stream);
  } else {
    if (ntiles >= 4 * 256 * 2) return run<BITS, MODE, 2, XL, EPI>(a, stream);
    return run<BITS, MODE, 1, XL, EPI>(a, stream);
  }
}

// Activation slice rows.  Up to K = 5120 (five k-blocks per wave): 8 rows for T = 5..8 and for
// the SwiGLU pair at T <= 4 (its two-tile workgroups run best with the register-free slice and
// the full ring: 24.6 against 25.3 us at T = 1), 16 rows for T = 9..16 (SwiGLU pair, T = 16:
// 36.5 against 44.9 us with fragments in the ring).  Otherwise 4 rows for T <= 4 and fragments
// in the ring above.
template <int BITS, int MODE, int EPI>
hipError_t pick_xl(const KArgs& a, hipStream_t stream) {
  const int nbw = (a.KB + kNW - 1) / kNW;
  if constexpr (MODE == MODE_MFMA) {
    if (nbw <= 5) {
      if (a.T <= 8 && (a.T > 4 || EPI == EPI_SWIGLU)) return pick_rt<BITS, MODE, 8, EPI>(a, stream);
      if (a.T > 8 && a.T <= 16) return pick_rt<BITS, MODE, 16, EPI>(a, stream);
    }
  }
  if (a.T <= 4) return pick_rt<BITS, MODE, 4, EPI>(a, stream);
  if constexpr (MODE == MODE_MFMA) return pick_rt<BITS, MODE, 0, EPI>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace

// This file is compiled once per code width and epilogue (W4_STREAM_BITS, W4_STREAM_EPI), so
// that the build compiles the six sets of kernel instances in parallel; each object defines the
// two launchers of its part, and kernels.h dispatches between them.
#if !defined(W4_STREAM_BITS) || !defined(W4_STREAM_EPI)
#error "compile with -DW4_STREAM_BITS=4|5 -DW4_STREAM_EPI=0|1|2"
#endif
#define W4_PART_NAME2(f, b, e) f##_b##b##_e##e
#define W4_PART_NAME(f, b, e) W4_PART_NAME2(f, b, e)

hipError_t W4_PART_NAME(launch_gemv, W4_STREAM_BITS, W4_STREAM_EPI)(const KArgs& a, hipStream_t stream) {
  return pick_xl<W4_STREAM_BITS, MODE_DOT2, W4_STREAM_EPI>(a, stream);
}

hipError_t W4_PART_NAME(launch_stream16, W4_STREAM_BITS, W4_STREAM_EPI)(const KArgs& a, hipStream_t stream) {
  return pick_xl<W4_STREAM_BITS, MODE_MFMA, W4_STREAM_EPI>(a, stream);
}

// 32- and 64-token modes (ring of 32- / 64-row activation tiles): K <= 5120 only
hipError_t W4_PART_NAME(launch_stream32, W4_STREAM_BITS, W4_STREAM_EPI)(const KArgs& a, hipStream_t stream) {
  if ((a.KB + kNW - 1) / kNW > 5) return hipErrorInvalidValue;
  return pick_rt<W4_STREAM_BITS, MODE_MFMA, 32, W4_STREAM_EPI>(a, stream);
}

hipError_t W4_PART_NAME(launch_stream64, W4_STREAM_BITS, W4_STREAM_EPI)(const KArgs& a, hipStream_t stream) {
  if ((a.KB + kNW - 1) / kNW > 5) return hipErrorInvalidValue;
  return pick_rt<W4_STREAM_BITS, MODE_MFMA, 64, W4_STREAM_EPI>(a, stream);
}

#if W4_STREAM_BITS == 4 && W4_STREAM_EPI == 0
// Grouped launch (both code widths are compiled here).  The slice or ring mode follows the
// single-matrix choice for the same T at K <= 5120 (a 4-, 8- or 16-row slice up to 16 tokens,
// the 32- or 64-row ring up to 64), so every output is bit-identical to the single-matrix
// call's; the row tiles per workgroup are chosen for the group as a whole (launch_grouped).
namespace {
template <int RT, int XL, int KPW>
hipError_t run_grouped_k(const GroupedArgs& ga, hipStream_t stream) {
  GArgs g;
  g.n = ga.n;
  int total = 0;
  for (int p = 0; p < ga.n; ++p) {
    g.a[p] = ga.a[p];
    g.bits[p] = ga.bits[p];
    total += (ga.a[p].rows / 16 + RT - 1) / RT;
    g.end[p] = total;
  }
  const KArgs& a = ga.a[0];
  const int nbw = (a.KB + kNW - 1) / kNW;
  const int nbc = nbw < KPW ? nbw : KPW;
  constexpr bool DMA = slice_dma<XL, KPW, false>();
  const int xdim = DMA ? nbc : nbc * 128 + 8;
  const size_t lds = stream_lds<MODE_MFMA, RT, XL, DMA>(nbc, xdim);
  constexpr int D = ring_depth<RT, XL, KPW>();
  if (a.K % 128)
    return launch_kernel(&stream_grouped_kernel<MODE_MFMA, RT, kNW, KPW, D, XL, EPI_STORE, false, true>,
                         dim3(total), dim3(kNW * 64), lds, stream, g, xdim);
  return launch_kernel(&stream_grouped_kernel<MODE_MFMA, RT, kNW, KPW, D, XL, EPI_STORE, false, false>,
                       dim3(total), dim3(kNW * 64), lds, stream, g, xdim);
}

template <int RT, int XL>
hipError_t run_grouped(const GroupedArgs& ga, hipStream_t stream) {
  switch ((ga.a[0].KB + kNW - 1) / kNW) {
    case 1: return run_grouped_k<RT, XL, 1>(ga, stream);
    case 2: return run_grouped_k<RT, XL, 2>(ga, stream);
    case 3: return run_grouped_k<RT, XL, 3>(ga, stream);
    case 4: return run_grouped_k<RT, XL, 4>(ga, stream);
    case 5: return run_grouped_k<RT, XL, 5>(ga, stream);
    default: return hipErrorInvalidValue;  // K <= 5120 only
  }
}

}  // namespace

// Row tiles per workgroup: at T <= 4 one (as the single-matrix route); otherwise the count
// tiles_per_workgroup picks for the group as a whole, with the start-up cost of a slice or of a
// ring, and at most two with the 64-row ring (whose 5-bit body, compiled into the same kernel,
// cannot hold three tiles' accumulators).  A group's matrices rarely divide into whole rounds
// the way one matrix does: 4-bit 4096 + 5-bit 12288 rows with three tiles is 342 workgroups, so
// 86 compute units run two and the launch waits for them (T = 8: 20.1 us), while two tiles make
// 512, two per compute unit (15.1 us).
hipError_t launch_grouped(const GroupedArgs& ga, hipStream_t stream) {
  if (ga.n < 1 || ga.n > kMaxParents) return hipErrorInvalidValue;
  const int T = ga.a[0].T;
  if (T < 1 || T > 64) return hipErrorInvalidValue;
  if (T <= 4) return run_grouped<1, 4>(ga, stream);
  TileGroup m[kMaxParents];
  for (int p = 0; p < ga.n; ++p) m[p] = TileGroup{ga.a[p].rows / 16, ga.bits[p]};
  if (T <= 16) {
    const int rt = tiles_per_workgroup(m, ga.n, 3, 2);
    if (T <= 8) {
      if (rt == 1) return run_grouped<1, 8>(ga, stream);
      return rt == 2 ? run_grouped<2, 8>(ga, stream) : run_grouped<3, 8>(ga, stream);
    }
    if (rt == 1) return run_grouped<1, 16>(ga, stream);
    return rt == 2 ? run_grouped<2, 16>(ga, stream) : run_grouped<3, 16>(ga, stream);
  }
  if (T <= 32) {
    const int rt = tiles_per_workgroup(m, ga.n, 3, 6);
    if (rt == 1) return run_grouped<1, 32>(ga, stream);
    return rt == 2 ? run_grouped<2, 32>(ga, stream) : run_grouped<3, 32>(ga, stream);
  }
  const int rt = tiles_per_workgroup(m, ga.n, 2, 6);
  return rt == 1 ? run_grouped<1, 64>(ga, stream) : run_grouped<2, 64>(ga, stream);
}
#endif

}  // namespace w4
