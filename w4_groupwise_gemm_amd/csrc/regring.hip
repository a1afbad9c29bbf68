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
// Its 32-row form (regring32_kernel, further below) runs 32x32x16 steps on tile pairs with the
// activation blocks in a per-wave LDS ring instead of registers, and where pairs are few and K
// long splits K over the workgroups of a pair group, the last of them adding the partial sums.
#include "device.h"
#include "kernels.h"
#include "tile32.h"
#include <utility>

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
constexpr int kMaxSlices = 4;        // K slices of a pair group (32-row form)

struct RegPart {
  int units;  // units of `ut` row tiles in the matrix
  int ut;     // 1, or 2 for the SwiGLU op (gate tile 2 p, up tile 2 p + 1)
};

// K split over the workgroups of a pair group: fp32 partial sums of every workgroup, one arrival
// counter per group (slices = 1: no split)
struct SplitArgs {
  float* part;
  int* cnt;
  int slices;
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

// ---- The 32-row form (T up to 32 or 64): the same workgroup shape on 32-row tile pairs and
// 32x32x16 steps, which on this chip sustain about three times the rate of 16x16x32 steps from one
// wave per SIMD (measured: 2.2 against 0.54-0.76 PFLOP/s).  A 32x32x16 B fragment spans 32 token
// rows, 32 bytes each: read straight from X that would be 32 half-used L2 lines per instruction,
// so each wave streams its blocks' activation rows whole (four rows of 256 bytes per instruction)
// straight into a two-slot LDS ring of its own (XOR-swizzled 16-byte chunks, one array per slot)
// and reads the fragments from there; only the code words go through registers.  One pair per
// workgroup at up to 20 tokens runs eight waves (two per SIMD: twice the loads in flight).
//
// K split.  Where pairs are few and K is long (5120-row matrices: 160 pairs for 256 compute
// units) the workgroups of a pair group take S contiguous K slices (S = 2..4, chosen from the
// shape so that the largest share of pairs x k-blocks is smallest).  Each writes its fp32 sums
// to a workspace with device-coherent stores, waits for them, and counts itself in the group's
// counter; the last of the S adds the slices in slice order (bitwise reproducible whatever the
// arrival order), runs the epilogue and resets the counter.  No workgroup waits for another.
//
// Load order and waits.  The compiler places the waits for code registers (counting the
// direct-to-LDS loads issued after a code block, so such a wait leaves them in flight); the wait
// for an activation block is explicit.  Sub-step j runs: the wait for code block j (forced here,
// before anything else is issued: activation block j and code block j + 1 stay in flight), the
// refill of activation slot (j + 1) % 2, code block j + 2, then the explicit wait for activation
// block j (code block j + 1, activation block j + 1 and code block j + 2 may still be in flight),
// and the math.

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled whatever the body's size (a plain loop
// over pairs stays rolled for four or five pairs and sends the register arrays to scratch memory).
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

// one 16-byte direct-to-LDS load per lane (a device function: the host pass of a kernel that
// makes this call from a generic lambda drops the kernel's launch stub)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

template <int BITS, int NP>
struct Codes32 {
  u32x4 cw[NP][2];
  uint32_t hw[NP][2], sp[NP], zp[NP];
};

template <int BITS, int NW, int NTT, int NP, int EPI>
__global__ __launch_bounds__(NW * 64) void regring32_kernel(KArgs a, RegPart part, SplitArgs ws) {
  constexpr int BLK = block_bytes(BITS);
  constexpr int XR = 32 * NTT;              // activation rows per block
  constexpr int XB = XR * 256;              // bytes of one slot of one wave
  constexpr int NC = NP * (BITS == 5 ? 6 : 4);  // loads of one code block
  constexpr int NX = 8 * NTT;                   // loads of one activation block
  __shared__ __attribute__((aligned(16))) char xring0[NW * XB], xring1[NW * XB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // workgroup b takes K slice b % S of pair group b / S
  const int S = ws.slices, grp = blockIdx.x / S, slc = blockIdx.x - grp * S, G = gridDim.x / S;
  const int u0 = (int)((long long)grp * part.units / G);
  const int u1 = (int)((long long)(grp + 1) * part.units / G);
  const int pair0 = u0, np = u1 - u0;  // units are tile pairs
  const int ntiles = a.rows / 16;
  const int kb0 = (int)((long long)slc * a.KB / S), nkb = (int)((long long)(slc + 1) * a.KB / S) - kb0;
  const int nbw = wave < nkb ? (nkb - wave + NW - 1) / NW : 0;
  const int T = a.T;
  const auto Rw = rsrc(a.w, (uint32_t)((size_t)ntiles * a.KB * BLK));
  const uint32_t szbytes = (uint32_t)((size_t)ntiles * a.KB * a.szw * 4);
  const auto Rs = rsrc(a.sc, szbytes);
  const auto Rz = rsrc(a.zr, szbytes);
  const auto Rx = rsrc(a.x, (uint32_t)((size_t)T * a.K * 2));
  const auto R0 = rsrc(a.x, 0);
  const t32::LaneMap m = t32::lane_map(a, lane);
  // activation load j moves rows 4 j .. 4 j + 3 (lane l: row 4 j + l / 16, stored at chunk
  // l % 16, which holds source chunk (l % 16) ^ (row % 16)); rows at or beyond T start at 2^31,
  // past the end of any X; xoffh: the same with the chunks of columns 64 .. 127 past the end too
  // (a half-size last block)
  int xoff[NX], xoffh[NX];
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    const int t = 4 * j + (lane >> 4), sc = (lane & 15) ^ (t & 15);
    xoff[j] = t < T ? (t * a.K + sc * 8) * 2 : (int)0x80000000u;
    xoffh[j] = sc >= 8 ? (int)0x80000000u : xoff[j];
  }
  const int brow = lane & 31;
  const int bsw = brow * 256 + 16 * ((4 * (lane >> 5)) ^ (brow & 15));
  const uint32_t magic = vgpr_const(0x64006400u);
  const int rot = nbw > 0 ? (int)(blockIdx.x >> 3) % nbw : 0;
  auto kblock = [&](int i) __attribute__((always_inline)) { return kb0 + wave + NW * (i + rot < nbw ? i + rot : i + rot - nbw); };
  const bool full = np == NP;  // shares differ by at most one pair: only the last may be absent

  auto issue_codes = [&](Codes32<BITS, NP>& C, int i) __attribute__((always_inline)) {
    const bool ok = i < nbw;
    const int kb = ok ? kblock(i) : wave;
    const auto Rwb = ok ? Rw : R0, Rsb = ok ? Rs : R0, Rzb = ok ? Rz : R0;
    const auto Rwl = ok && full ? Rw : R0, Rsl = ok && full ? Rs : R0, Rzl = ok && full ? Rz : R0;
    unroll<NP>([&](auto pc) __attribute__((always_inline)) {
      constexpr int p = decltype(pc)::value;
      constexpr bool last = p == NP - 1;
      // the lane's tile of the pair (an odd tile count leaves the last pair without its second
      // tile: those lanes re-read the first, whose rows there are never stored)
      const int tile = min(2 * (pair0 + p) + m.th, ntiles - 1);
      const int bo = (tile * a.KB + kb) * BLK;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        C.cw[p][q] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(last ? Rwl : Rwb, bo + m.slot16[q], 0, kNT));
        if constexpr (BITS == 5)
          C.hw[p][q] = __builtin_amdgcn_raw_buffer_load_b32(last ? Rwl : Rwb, bo + 1024 + m.slot16[q] / 4, 0, kNT);
        else
          C.hw[p][q] = 0;
      }
      const int so = (tile * a.KB + kb) * a.szw * 4 + m.szoff;
      C.sp[p] = __builtin_amdgcn_raw_buffer_load_b32(last ? Rsl : Rsb, so, 0, 0);
      C.zp[p] = __builtin_amdgcn_raw_buffer_load_b32(last ? Rzl : Rzb, so, 0, 0);
    });
  };
  // activation rows of local block i into slot i % 2 (SL) of this wave
  auto issue_x = [&](auto slc, int i) __attribute__((always_inline)) {
    constexpr int SL = decltype(slc)::value;
    char* const dst = (SL ? xring1 : xring0) + wave * XB;
    const bool ok = i < nbw;
    const int kb = ok ? kblock(i) : wave;
    const bool half = ok && kb * 128 + 64 >= a.K;
    const auto Rxb = ok ? Rx : R0;
#pragma unroll
    for (int j = 0; j < NX; ++j)
      dma16(Rxb, dst + j * 1024, half ? xoffh[j] : xoff[j], kb * 256);
  };

  f32x16 acc[NP][NTT];
  unroll<NP>([&](auto pc) __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[decltype(pc)::value][tt] = f32x16{};
  });

  // Math of one block: eight 16-column steps, each the B fragments of step I for every token
  // tile, then each pair's weight fragment of its code dword I / 2 of set I % 2 and its NTT
  // matrix-core steps.
  auto math = [&](const Codes32<BITS, NP>& C, const char* xs) __attribute__((always_inline)) {
    ZS zs[NP];
    unroll<NP>([&](auto pc) __attribute__((always_inline)) {
      constexpr int p = decltype(pc)::value;
      zs[p] = zs_terms(C.zp[p], C.sp[p]);
    });
    unroll<8>([&](auto ic) __attribute__((always_inline)) {
      constexpr int I = decltype(ic)::value, J = I >> 1, Q = I & 1;
      f16x8 B[NTT];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) B[tt] = t32::load_b1<I>(xs, bsw, tt);
      unroll<NP>([&](auto pc) __attribute__((always_inline)) {
        constexpr int p = decltype(pc)::value;
        const f16x8 A = wfrag_zs<BITS, J>(C.cw[p][Q][J], C.hw[p][Q], magic, zs[p]);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[p][tt] = mfma32(A, B[tt], acc[p][tt]);
      });
    });
  };

  // Code blocks ride two ahead in three register slots, activation blocks one ahead in two LDS
  // slots: a round of six sub-steps returns both to their first slots.
  Codes32<BITS, NP> C[3];
  issue_codes(C[0], 0);
  issue_x(std::integral_constant<int, 0>{}, 0);
  issue_codes(C[1], 1);
  auto sub = [&](auto sc, int j) __attribute__((always_inline)) {
    constexpr int S6 = decltype(sc)::value;
    // the wait for code block j, before anything else goes out (see above)
    asm volatile("" ::"v"(C[S6 % 3].zp[NP - 1]));
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt 0: the last block's fragment reads are done
    issue_x(std::integral_constant<int, (S6 + 1) % 2>{}, j + 1);
    issue_codes(C[(S6 + 2) % 3], j + 2);
    __builtin_amdgcn_sched_barrier(0);
    // activation block j has landed (code j + 1, x j + 1, code j + 2 may not); a wave never has
    // more than 63 loads outstanding, so with more behind block j it has landed already
    wait_vmcnt<(2 * NC + NX < 63 ? 2 * NC + NX : 63)>();
    math(C[S6 % 3], (S6 % 2 ? xring1 : xring0) + wave * XB);
    __builtin_amdgcn_sched_barrier(0);
  };
  int i0 = 0;
  for (; i0 + 6 <= nbw; i0 += 6) {
    sub(std::integral_constant<int, 0>{}, i0);
    sub(std::integral_constant<int, 1>{}, i0 + 1);
    sub(std::integral_constant<int, 2>{}, i0 + 2);
    sub(std::integral_constant<int, 3>{}, i0 + 3);
    sub(std::integral_constant<int, 4>{}, i0 + 4);
    sub(std::integral_constant<int, 5>{}, i0 + 5);
  }
  // a last partial round (the same sub-steps: their loads past the wave's last block read zeros)
  if (i0 < nbw) sub(std::integral_constant<int, 0>{}, i0);
  if (i0 + 1 < nbw) sub(std::integral_constant<int, 1>{}, i0 + 1);
  if (i0 + 2 < nbw) sub(std::integral_constant<int, 2>{}, i0 + 2);
  if (i0 + 3 < nbw) sub(std::integral_constant<int, 3>{}, i0 + 3);
  if (i0 + 4 < nbw) sub(std::integral_constant<int, 4>{}, i0 + 4);

  // ---- fixed-order combination of the four partial sums, pair by pair, then the epilogue.
  // red[w][tt][v][lane]: wave w's sums of the pair, token tile tt, accumulator register v (in
  // the first ring array, free once every wave has left the loop).
  static_assert(NW * NTT * 16 * 64 * 4 <= NW * XB, "reduction fits the first ring array");
  float* red = reinterpret_cast<float*>(xring0);
  wait_vmcnt<0>();
  auto combine = [&](auto pc) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    if (P >= np) return;  // (uniform over the workgroup)
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((wave * NTT + tt) * 16 + v) * 64 + lane] = acc[P][tt][v];
    __syncthreads();
    if (threadIdx.x < NTT * 64) {
      const int tt = threadIdx.x >> 6, l = threadIdx.x & 63;
      f32x16 sum;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = red[((0 * NTT + tt) * 16 + v) * 64 + l];
#pragma unroll
        for (int w = 1; w < NW; ++w) x += red[((w * NTT + tt) * 16 + v) * 64 + l];
        sum[v] = x;
      }
      if (S == 1) {
        t32::store_pair<EPI>(a, sum, pair0 + P, 32 * tt, ntiles, l);
      } else {
        float* dst = ws.part + ((size_t)(blockIdx.x * NP + P) * NTT + tt) * 1024 + l;
#pragma unroll
        for (int v = 0; v < 16; ++v)
          __hip_atomic_store(dst + v * 64, sum[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  unroll<NP>(combine);
  if (S == 1) return;
  // Arrival: the partial stores are device-coherent and complete (vmcnt 0 in every thread before
  // the barrier) when the workgroup is counted; the last of the group's S workgroups then reads
  // them back with device-coherent loads.  No cache-wide fence is needed (one costs far more than
  // the whole reduction on this chip).
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(ws.cnt + grp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
  __syncthreads();
  if (!last) return;
  // pair by pair: every thread adds its share of the pair's values over the slices in slice
  // order (all loads issued first) into the LDS, then the first NTT waves run the epilogue
  constexpr int EL = NTT * 1024, PER = EL / (NW * 64);
  for (int P = 0; P < np; ++P) {
    float v[kMaxSlices][PER];
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q)
#pragma unroll
      for (int j = 0; j < PER; ++j)
        v[q][j] = q < S ? __hip_atomic_load(ws.part + (size_t)((grp * S + q) * NP + P) * EL + threadIdx.x + NW * 64 * j,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : 0.f;
    __syncthreads();  // the previous pair's epilogue has read the LDS
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      float x = v[0][j];
#pragma unroll
      for (int q = 1; q < kMaxSlices; ++q)
        if (q < S) x += v[q][j];
      red[threadIdx.x + NW * 64 * j] = x;
    }
    __syncthreads();
    if (threadIdx.x < NTT * 64) {
      const int tt = threadIdx.x >> 6, l = threadIdx.x & 63;
      f32x16 sum;
#pragma unroll
      for (int u = 0; u < 16; ++u) sum[u] = red[(tt * 16 + u) * 64 + l];
      t32::store_pair<EPI>(a, sum, pair0 + P, 32 * tt, ntiles, l);
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(ws.cnt + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BITS, int NW, int NTT, int NP, int EPI>
hipError_t run32(const KArgs& a, int grid, RegPart part, SplitArgs sa, hipStream_t stream) {
  return launch_kernel(&regring32_kernel<BITS, NW, NTT, NP, EPI>, dim3(grid), dim3(NW * 64), 0, stream, a,
                       part, sa);
}

// Pair groups for S slices: one workgroup per compute unit (groups = min(units, 256 / S)), more
// only when a group would exceed five pairs; returns the largest group.
inline int groups_for(int units, int S, int* grid) {
  const int gmax = kCUs / S;
  int g = units < gmax ? units : gmax;
  if ((units + g - 1) / g > kMaxPairs) g = (units + kMaxPairs - 1) / kMaxPairs;
  *grid = g;
  return (units + g - 1) / g;
}

// Slices of K per pair group: the count whose largest workgroup share (pairs x k-blocks) is
// smallest, taken only when it is at most 4/5 of the unsplit share (the partial sums and the
// last workgroup's reduction cost about that at 64 k-blocks) and K has at least 64 blocks
// (5120-row matrices, measured: K = 8192 / 12288 / 17408 at 17-64 tokens 15-40 % faster with
// three slices; at K = 6144 the split gains nothing below 40 tokens).
inline int slices_for(int units, int KB) {
  if (KB < 64) return 1;
  int grid = 0;
  const long long base = (long long)groups_for(units, 1, &grid) * KB;
  int best = 1;
  long long cost = base;
  for (int S = 2; S <= kMaxSlices; ++S) {
    const long long c = (long long)groups_for(units, S, &grid) * ((KB + S - 1) / S);
    if (c < cost) {
      cost = c;
      best = S;
    }
  }
  return 5 * cost <= 4 * base ? best : 1;
}

// Pair groups spread evenly over one workgroup per compute unit (up to five pairs each); with a
// K split, S workgroups per group, each taking one contiguous K slice.  Without a workspace, or
// one too small for the partial sums, K stays whole.
template <int BITS, int NTT, int EPI>
hipError_t pick_np32(const KArgs& a, const SplitWs& ws, hipStream_t stream) {
  const int units = (a.rows / 16 + 1) / 2;
  int S = ws.part ? slices_for(units, a.KB) : 1;
  int grid = 0;
  int per = groups_for(units, S, &grid);
  if (S > 1 && (grid > ws.groups || (size_t)grid * S * per * NTT * 4096 > ws.part_bytes)) {
    S = 1;
    per = groups_for(units, 1, &grid);
  }
  const RegPart part{units, 2};
  const SplitArgs sa{ws.part, ws.cnt, S};
  grid *= S;
  // eight waves for a single pair per workgroup up to 20 tokens (more loads in flight per pair)
  if constexpr (NTT == 1)
    if (S == 1 && per == 1 && a.T <= 20) return run32<BITS, 8, 1, 1, EPI>(a, grid, part, sa, stream);
  switch (per) {
    case 1: return run32<BITS, 4, NTT, 1, EPI>(a, grid, part, sa, stream);
    case 2: return run32<BITS, 4, NTT, 2, EPI>(a, grid, part, sa, stream);
    case 3: return run32<BITS, 4, NTT, 3, EPI>(a, grid, part, sa, stream);
    case 4: return run32<BITS, 4, NTT, 4, EPI>(a, grid, part, sa, stream);
    default: return run32<BITS, 4, NTT, 5, EPI>(a, grid, part, sa, stream);
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

template <int BITS, int EPI>
hipError_t pick_ntt(int tn, const KArgs& a, const SplitWs& ws, hipStream_t stream) {
  if (a.T > tn) return hipErrorInvalidValue;
  return tn <= 32 ? pick_np32<BITS, 1, EPI>(a, ws, stream) : pick_np32<BITS, 2, EPI>(a, ws, stream);
}

template <int BITS>
hipError_t pick_epi32(int tn, int epi, const KArgs& a, const SplitWs& ws, hipStream_t stream) {
  if (epi == EPI_SWIGLU) return pick_ntt<BITS, EPI_SWIGLU>(tn, a, ws, stream);
  if (epi == EPI_ADD) return pick_ntt<BITS, EPI_ADD>(tn, a, ws, stream);
  return pick_ntt<BITS, EPI_STORE>(tn, a, ws, stream);
}

}  // namespace

// One object per code width (W4_REGRING_BITS), so that the two compile in parallel.
#if W4_REGRING_BITS == 4
hipError_t launch_regring_b4(int tn, int epi, const KArgs& a, hipStream_t stream) {
  return pick_epi<4>(tn, epi, a, stream);
}
hipError_t launch_regring32_b4(int tn, int epi, const KArgs& a, const SplitWs& ws, hipStream_t stream) {
  return pick_epi32<4>(tn, epi, a, ws, stream);
}
#elif W4_REGRING_BITS == 5
hipError_t launch_regring_b5(int tn, int epi, const KArgs& a, hipStream_t stream) {
  return pick_epi<5>(tn, epi, a, stream);
}
hipError_t launch_regring32_b5(int tn, int epi, const KArgs& a, const SplitWs& ws, hipStream_t stream) {
  return pick_epi32<5>(tn, epi, a, ws, stream);
}
#else
#error "compile regring.hip with -DW4_REGRING_BITS=4 or 5"
#endif

}  // namespace w4
