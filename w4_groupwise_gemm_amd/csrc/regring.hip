// Register-ring path for up to 64 tokens: every operand of the matrix-core steps is loaded
// straight into registers, a ring of k-blocks ahead of the math; LDS is used only for the final
// combination of the partial sums.
//
// Prior art: the small-T MMA kernels and shared activation slabs of the ninfer-3080 performance
// notes ("What changed"; "What is left at C1 / C8": at these widths the kernels are a streaming
// problem with a dequantisation tax, bounded by operand movement and occupancy).
//
// gfx950 design:
//  * one workgroup of four waves (one per SIMD) per compute unit; the row tiles are spread
//    evenly over the grid in units of one 16-row tile (one gate / up tile pair for the SwiGLU
//    op), so a launch is one round whose shares differ by at most one unit;
//  * the four waves split K (wave w takes k-blocks w, w + 4, ...) and each runs every row tile
//    of the workgroup on its blocks: each code byte and each activation byte the workgroup needs
//    is loaded once, by the lane that feeds it to the matrix core, and the activation matrix
//    crosses the L2 once per workgroup;
//  * per k-block a wave loads, for each row tile, one 16-byte code word per lane (5-bit codes:
//    plus the high-plane word) and its scale / zero-point words, and for each 16-token tile the
//    four 16-byte B fragments of the block's four 32-column steps straight from X (lane l: token
//    16 q + l % 16, the k slots of its own code dword); D blocks of these loads stay in flight
//    ahead of the math, and since all of them are register loads on the wave's one in-order
//    counter, every wait the compiler inserts is exact;
//  * loads past a wave's last block, of row tiles past the workgroup's share and of the empty
//    half of a half-size last block go through an empty buffer resource, and those of token rows
//    at or beyond T through an offset past the end of X: they return zeros, move no data and keep
//    the load count of every block the same, and their zeros add nothing to the sums;
//  * the dequantisation is the magic-bias decode in 13 vector ops per packed word for any
//    zero-point (its integer part taken off exactly with the bias, its fraction folded into the
//    scale step), so each block's math is one branch-free sequence; each weight fragment feeds
//    one 16x16x32 matrix-core step per 16-token tile;
//  * the four partial sums are combined in LDS in a fixed order (bitwise deterministic), then the
//    store / SwiGLU / add epilogue.
#include "device.h"
#include "kernels.h"
#include "tile32.h"

namespace w4 {
namespace {

using namespace w4dev;
using t32::rsrc;
using t32::wfrag;
using w4layout::block_bytes;

constexpr int kNW = 4;               // waves per workgroup, one per SIMD
constexpr int kCUs = 256;            // compute units of the chip (gfx950, MI350 series)
constexpr int kMaxTiles = 6;         // row tiles per workgroup, single matrices
constexpr int kMaxPairs = 5;         // gate / up tile pairs per workgroup, SwiGLU op
constexpr int kNT = 2;               // cache policy of the code loads: non-temporal (read once)

struct RegPart {
  int units;  // units of `ut` row tiles in the matrix
  int ut;     // 1, or 2 for the SwiGLU op (gate tile 2 p, up tile 2 p + 1)
};

// Loads of one k-block for one wave: RT row tiles of codes and TQ 16-token tiles of activations.
template <int BITS, int RT, int TQ>
struct Slot {
  u32x4 cw[RT];
  uint32_t hw[RT], sp[RT], zp[RT];
  u32x4 xb[TQ][4];
};

// Zero-point and scale terms of one (row tile, k-block) for this lane, both groups of the block
// as fp16 pairs.  z = zi + zf with zi = round(z): 1024 + zi and 64 + zi are exact, so the bias and
// zi come off in one exact packed add (or fma), and w = (q - zi) s - zf s in one packed fma.
// Integer zero-points (zf = 0) give fp16((q - z) s) exactly, as the other kernels; a fractional
// one adds one rounding, of zf s (below 2^-12 s).  No branch: one code path for every block.
struct ZS {
  f16x2 nb0, nb1, s, c;  // -(1024 + zi), -(64 + zi), s, -zf s
};
__device__ __forceinline__ ZS zs_terms(uint32_t zp, uint32_t sp) {
  const f16x2 z = as_h2(zp), s = as_h2(sp);
  const f16x2 c1024 = {(f16)1024.0f, (f16)1024.0f}, c960 = {(f16)960.0f, (f16)960.0f};
  const f16x2 nb0 = -(z + c1024);
  const f16x2 zf = z - ((-nb0) - c1024);
  return ZS{nb0, nb0 + c960, s, -(zf * s)};
}

// fp16 weights of packed dword J (8 k slots of the lane's row) from the biased pairs.
template <int BITS, int J>
__device__ __forceinline__ f16x8 wfrag_zs(uint32_t w, uint32_t hiw, uint32_t magic, const ZS& t) {
  uint32_t u[4];
  wbiased<BITS, J>(w, hiw, magic, u);
  constexpr int H = J >> 1;  // group of the dword
  const f16x2 b0 = __builtin_shufflevector(t.nb0, t.nb0, H, H);
  const f16x2 b1 = __builtin_shufflevector(t.nb1, t.nb1, H, H);
  const f16x2 s2 = __builtin_shufflevector(t.s, t.s, H, H);
  const f16x2 c2 = __builtin_shufflevector(t.c, t.c, H, H);
  const f16x2 c16th = {(f16)0.0625f, (f16)0.0625f};
  return cat8((as_h2(u[0]) + b0) * s2 + c2, (as_h2(u[1]) * c16th + b1) * s2 + c2,
              (as_h2(u[2]) + b0) * s2 + c2, (as_h2(u[3]) * c16th + b1) * s2 + c2);
}

// Ring depth: as many blocks in flight as the registers hold (one slot is RT (7 or 8) + 16 TQ
// registers; the accumulators take 4 RT TQ, mostly in the second register file, and about 48
// go to addresses and the dequantised fragments, of 480 usable) and as the wave's load counter
// counts (63 outstanding loads; a block issues 3 or 4 per row tile and 4 per token tile).
template <int BITS, int RT, int TQ>
constexpr int ring_depth() {
  constexpr int slot = RT * (BITS == 5 ? 8 : 7) + 16 * TQ;
  constexpr int by_regs = (480 - 4 * RT * TQ - 48) / slot - 1;
  constexpr int by_count = 63 / (RT * (BITS == 5 ? 4 : 3) + 4 * TQ);
  constexpr int d = by_regs < by_count ? by_regs : by_count;
  return d < 1 ? 1 : d > 4 ? 4 : d;
}

template <int BITS, int TQ, int RT, int D, int EPI>
__global__ __launch_bounds__(kNW * 64) void regring_kernel(KArgs a, RegPart part) {
  constexpr int BLK = block_bytes(BITS);
  constexpr int NS = D + 1;  // ring slots: D blocks in flight while one is consumed
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int u0 = (int)((long long)blockIdx.x * part.units / gridDim.x);
  const int u1 = (int)((long long)(blockIdx.x + 1) * part.units / gridDim.x);
  const int tile0 = u0 * part.ut, nt = (u1 - u0) * part.ut;
  const int ntiles = a.rows / 16;
  const int nbw = wave < a.KB ? (a.KB - wave + kNW - 1) / kNW : 0;
  const int T = a.T;
  const auto Rw = rsrc(a.w, (uint32_t)((size_t)ntiles * a.KB * BLK));
  const uint32_t szbytes = (uint32_t)((size_t)ntiles * a.KB * a.szw * 4);
  const auto Rs = rsrc(a.sc, szbytes);
  const auto Rz = rsrc(a.zr, szbytes);
  const auto Rx = rsrc(a.x, (uint32_t)((size_t)T * a.K * 2));
  const auto R0 = rsrc(a.x, 0);  // empty: every load through it returns zero
  // Lane parts of the offsets (the block and tile parts are wave-uniform scalars).  X: token
  // 16 q + r, column 16 g of a block; token rows at or beyond T start at 2^31, past the end of
  // any X (the scalar and immediate parts stay below 2^31, so the sum cannot wrap).
  const int cofs = lane * 16, hofs = lane * 4, szoff = 4 * sz_lane_word(a, r, g);
  int xoff[TQ];
#pragma unroll
  for (int q = 0; q < TQ; ++q) {
    const int t = 16 * q + r;
    xoff[q] = t < T ? (t * a.K + 16 * g) * 2 : (int)0x80000000u;
  }
  const uint32_t magic = vgpr_const(0x64006400u);

  // Loads of local block i (k-block wave + 4 i) into slot S.  Blocks past the wave's last one
  // and row tiles past the workgroup's share read through the empty resource (zeros, no
  // traffic), so that every slot is consumed by the same math and every wait stays exact.
  constexpr int UT = EPI == EPI_SWIGLU ? 2 : 1;
  const bool full = nt == RT;  // shares differ by at most one unit: only the last may be absent
  // Each workgroup starts its waves' block sequences at its own offset.  At K = 5120 an
  // activation row is 80 L2 lines long, so the 64 rows of one k-block sit in the same few L2
  // channels; workgroups that walked k in step would all queue on those channels at once.
  // (Workgroups of one XCD are 8 apart in launch order.)
  const int rot = nbw > 0 ? (int)(blockIdx.x >> 3) % nbw : 0;
  auto issue = [&](Slot<BITS, RT, TQ>& S, int i) {
    const bool ok = i < nbw;
    const int ir = i + rot < nbw ? i + rot : i + rot - nbw;
    const int kb = wave + kNW * (ok ? ir : i);
    const bool half = kb * 128 + 64 >= a.K;  // only group 0 of this block is real
    const auto Rwb = ok ? Rw : R0, Rsb = ok ? Rs : R0, Rzb = ok ? Rz : R0;
    const auto Rwl = ok && full ? Rw : R0, Rsl = ok && full ? Rs : R0, Rzl = ok && full ? Rz : R0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const bool last = rt >= RT - UT;
      const int bi = (tile0 + rt) * a.KB + kb;
      S.cw[rt] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(last ? Rwl : Rwb, cofs, bi * BLK, kNT));
      if constexpr (BITS == 5)
        S.hw[rt] = __builtin_amdgcn_raw_buffer_load_b32(last ? Rwl : Rwb, hofs, bi * BLK + 1024, kNT);
      else
        S.hw[rt] = 0;
      S.sp[rt] = __builtin_amdgcn_raw_buffer_load_b32(last ? Rsl : Rsb, szoff, bi * a.szw * 4, 0);
      S.zp[rt] = __builtin_amdgcn_raw_buffer_load_b32(last ? Rzl : Rzb, szoff, bi * a.szw * 4, 0);
    }
    const auto Rx0 = ok ? Rx : R0, Rx1 = ok && !half ? Rx : R0;
#pragma unroll
    for (int q = 0; q < TQ; ++q) {
#pragma unroll
      for (int J = 0; J < 4; ++J)
        S.xb[q][J] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(J < 2 ? Rx0 : Rx1, xoff[q],
                                                         kb * 256 + (64 * (J >> 1) + 8 * (J & 1)) * 2, 0));
    }
  };

  f32x4 acc[RT][TQ];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int q = 0; q < TQ; ++q) acc[rt][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Math of one slot.
  auto math = [&](const Slot<BITS, RT, TQ>& S) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const ZS t = zs_terms(S.zp[rt], S.sp[rt]);
      f16x8 A[4];
      A[0] = wfrag_zs<BITS, 0>(S.cw[rt][0], S.hw[rt], magic, t);
      A[1] = wfrag_zs<BITS, 1>(S.cw[rt][1], S.hw[rt], magic, t);
      A[2] = wfrag_zs<BITS, 2>(S.cw[rt][2], S.hw[rt], magic, t);
      A[3] = wfrag_zs<BITS, 3>(S.cw[rt][3], S.hw[rt], magic, t);
#pragma unroll
      for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int q = 0; q < TQ; ++q) acc[rt][q] = mfma16(A[J], __builtin_bit_cast(f16x8, S.xb[q][J]), acc[rt][q]);
    }
  };

  // The ring: slot s of round i0 holds block i0 + s.  Full rounds run branch-free (every wait
  // the compiler places is then exact); the blocks of a last, partial round were issued by the
  // rounds before it and are consumed after the loop.
  Slot<BITS, RT, TQ> S[NS];
#pragma unroll
  for (int s = 0; s < D; ++s) issue(S[s], s);
  int i0 = 0;
  for (; i0 + NS <= nbw; i0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      // the refill goes out before the block's math (the scheduler would otherwise sink the
      // loads into the math to save registers, and the ring would run without a block ahead)
      issue(S[(s + D) % NS], i0 + s + D);
      __builtin_amdgcn_sched_barrier(0);
      math(S[s]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < nbw - i0) math(S[s]);

  // ---- fixed-order combination of the four partial sums, PT row tiles at a time, then the
  // epilogue.  red[w][k][q][lane]: wave w's sums of tile p0 + k, token tile q.
  extern __shared__ __attribute__((aligned(16))) char smem[];
  f32x4* red = reinterpret_cast<f32x4*>(smem);
  constexpr int PT = EPI == EPI_SWIGLU ? 2 : RT;
  static_assert(RT % PT == 0, "passes of whole units");
#pragma unroll
  for (int p0 = 0; p0 < RT; p0 += PT) {
    if (p0 >= nt) break;  // (uniform over the workgroup)
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PT; ++k)
#pragma unroll
      for (int q = 0; q < TQ; ++q) red[((wave * PT + k) * TQ + q) * 64 + lane] = acc[p0 + k][q];
    __syncthreads();
    constexpr int ITEMS = TQ * (PT / UT) * 64;
    for (int it = threadIdx.x; it < ITEMS; it += kNW * 64) {
      const int l = it & 63, q = (it >> 6) % TQ, u = (it >> 6) / TQ;
      const int t = 16 * q + (l & 15);
      const int rt = p0 + u * UT;
      if (t >= T || rt >= nt) continue;
      auto sum = [&](int k) {
        f32x4 v = red[(k * TQ + q) * 64 + l];
        for (int w = 1; w < kNW; ++w) v = v + red[((w * PT + k) * TQ + q) * 64 + l];
        return v;
      };
      if constexpr (EPI == EPI_SWIGLU)
        store_quad<EPI>(a, t, ((tile0 + rt) >> 1) * 16 + 4 * (l >> 4), sum(u * 2), sum(u * 2 + 1));
      else
        store_quad<EPI>(a, t, (tile0 + rt) * 16 + 4 * (l >> 4), sum(u), f32x4{});
    }
  }
}

template <int BITS, int TQ, int RT, int EPI>
hipError_t run(const KArgs& a, int grid, RegPart part, hipStream_t stream) {
  constexpr int D = ring_depth<BITS, RT, TQ>();
  constexpr int PT = EPI == EPI_SWIGLU ? 2 : RT;
  const size_t lds = (size_t)kNW * PT * TQ * 1024;
  return launch_kernel(&regring_kernel<BITS, TQ, RT, D, EPI>, dim3(grid), dim3(kNW * 64), lds, stream,
                       a, part);
}

// One workgroup per compute unit (fewer when there are fewer units), each with an even share of
// the units; more workgroups only when a share would exceed the largest instance.
template <int BITS, int TQ, int EPI>
hipError_t pick_rt(const KArgs& a, hipStream_t stream) {
  const int ut = EPI == EPI_SWIGLU ? 2 : 1;
  const int units = a.rows / 16 / ut;
  const int cap = EPI == EPI_SWIGLU ? kMaxPairs : kMaxTiles;  // units per workgroup
  int grid = units < kCUs ? units : kCUs;
  if ((units + grid - 1) / grid > cap) grid = (units + cap - 1) / cap;
  const int per = (units + grid - 1) / grid;  // largest share
  const RegPart part{units, ut};
  if constexpr (EPI == EPI_SWIGLU) {
    switch (per) {
      case 1: return run<BITS, TQ, 2, EPI>(a, grid, part, stream);
      case 2: return run<BITS, TQ, 4, EPI>(a, grid, part, stream);
      case 3: return run<BITS, TQ, 6, EPI>(a, grid, part, stream);
      case 4: return run<BITS, TQ, 8, EPI>(a, grid, part, stream);
      default: return run<BITS, TQ, 10, EPI>(a, grid, part, stream);
    }
  } else {
    switch (per) {
      case 1: return run<BITS, TQ, 1, EPI>(a, grid, part, stream);
      case 2: return run<BITS, TQ, 2, EPI>(a, grid, part, stream);
      case 3: return run<BITS, TQ, 3, EPI>(a, grid, part, stream);
      case 4: return run<BITS, TQ, 4, EPI>(a, grid, part, stream);
      case 5: return run<BITS, TQ, 5, EPI>(a, grid, part, stream);
      default: return run<BITS, TQ, 6, EPI>(a, grid, part, stream);
    }
  }
}

template <int BITS, int EPI>
hipError_t pick_tq(int tn, const KArgs& a, hipStream_t stream) {
  if (a.T > tn) return hipErrorInvalidValue;
  if (tn <= 16) return pick_rt<BITS, 1, EPI>(a, stream);
  if (tn <= 32) return pick_rt<BITS, 2, EPI>(a, stream);
  return pick_rt<BITS, 4, EPI>(a, stream);
}

template <int BITS>
hipError_t pick_epi(int tn, int epi, const KArgs& a, hipStream_t stream) {
  if (epi == EPI_SWIGLU) return pick_tq<BITS, EPI_SWIGLU>(tn, a, stream);
  if (epi == EPI_ADD) return pick_tq<BITS, EPI_ADD>(tn, a, stream);
  return pick_tq<BITS, EPI_STORE>(tn, a, stream);
}

}  // namespace

// One object per code width (W4_REGRING_BITS), so that the two compile in parallel.
#if W4_REGRING_BITS == 4
hipError_t launch_regring_b4(int tn, int epi, const KArgs& a, hipStream_t stream) {
  return pick_epi<4>(tn, epi, a, stream);
}
#elif W4_REGRING_BITS == 5
hipError_t launch_regring_b5(int tn, int epi, const KArgs& a, hipStream_t stream) {
  return pick_epi<5>(tn, epi, a, stream);
}
#else
#error "compile regring.hip with -DW4_REGRING_BITS=4 or 5"
#endif

}  // namespace w4
