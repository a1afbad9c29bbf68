// Wide matrix-core path: prefill widths (hundreds to thousands of token columns).
//
// Prior art: the prefill schedules of the ninfer-3080 performance notes ("The token tile, and
// why it was hiding": a token tile of BN columns re-streams the whole weight matrix T/BN times,
// so the tile must be wide; "What is still missing": the mainloop -- double buffering and a
// conflict-free shared layout).
//
// gfx950 design.
//  * The matrix-core step is v_mfma_f32_32x32x16_f16 (on this chip it sustains about twice the
//    rate of the 16x16x32 form).  Its A operand is a 32-row "pair" of two 16-row packed tiles:
//    a lane of the instruction takes row l%32 and k half l/32, and that is exactly what one
//    16-byte load per lane from the packed layout delivers when the 16-lane groups of the two
//    tiles are picked in the order (tile a, tile b, tile a, tile b): no repacking and no lane
//    shuffles.  The four dwords of that load are four 16-k steps.  Weights never touch LDS;
//    they are dequantised in registers, 13 (4-bit) or 19 (5-bit) vector ops per dword.
//  * Workgroup = 4 waves.  Wave w owns pair w for every token tile of the workgroup, so each
//    dequantised fragment feeds NTT matrix-core steps.  5120-row projections use 160-row
//    workgroups (32 of them tile N exactly); the fifth pair is split between the four waves by
//    k step (each wave does two of its eight steps per block for all token tiles), and the
//    four partial sums are added in a fixed order through LDS at the end, so no wave
//    dequantises more than a quarter of it and results stay bitwise reproducible.
//  * The activation tile X[BN tokens][128 columns] of each k-block is loaded straight into LDS
//    with buffer_load ... lds (no register staging), double buffered, one barrier per k-block.
//    16-byte chunks are stored XOR-swizzled by token row (chunk c of row r sits at c ^ (r & 15)),
//    so the 16 lanes of a read phase hit 16 distinct bank groups.
//  * Tiles are ordered so that the workgroups running at the same time on one XCD (round-robin
//    dispatch) cover all row blocks of the same token block: that activation tile is fetched
//    into the XCD's L2 once and shared, instead of being re-read per row block.
//  * Integer zero-points (checked exactly, once per workgroup) take the short dequantisation;
//    fractional ones the general form.
#include "device.h"
#include "kernels.h"
#include "tile32.h"

namespace w4 {
namespace {

using namespace w4dev;
using namespace t32;
using w4layout::block_bytes;

// The share of the fifth pair that one wave computes: its two dwords (k-steps) of one set.
template <int BITS>
struct ShareCodes {
  u32x2 cw;
  uint32_t hw;
  uint32_t sp, zp;
};

// Wave W's share of pair `pair`: set S = W / 2, dwords j = 2 (W % 2) and 2 (W % 2) + 1.
template <int BITS, int W>
__device__ __forceinline__ void load_share(ShareCodes<BITS>& c, const Rsrcs& R, const KArgs& a,
                                           const LaneMap& m, int pair, int ntiles, int kb) {
  constexpr int BLK = block_bytes(BITS);
  const int tile = min(2 * pair + m.th, ntiles - 1);
  const int bi = tile * a.KB + kb;
  const int slot = m.slot16[W >> 1];
  c.cw = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(R.w, bi * BLK + slot + 8 * (W & 1), 0, 0));
  if constexpr (BITS == 5)
    c.hw = __builtin_amdgcn_raw_buffer_load_b32(R.w, bi * BLK + 1024 + slot / 4, 0, 0);
  else
    c.hw = 0;
  c.sp = __builtin_amdgcn_raw_buffer_load_b32(R.s, bi * 4 * a.szw + m.szoff, 0, 0);
  c.zp = __builtin_amdgcn_raw_buffer_load_b32(R.z, bi * 4 * a.szw + m.szoff, 0, 0);
}

// k-steps of a block, in group order: index i = 2 J + S is the 16-k step (J, S); steps 0..3
// cover group 0 of the block and steps 4..7 group 1, which a half-empty last block
// (K % 128 == 64) does not have.  Wave W's share of the fifth pair is the set S = W / 2 of
// dwords J = 2 (W % 2) and 2 (W % 2) + 1.
template <int NP, int W, int I>
constexpr bool share_step() {
  return NP == 5 && (I & 1) == (W >> 1) && ((I >> 1) >> 1) == (W & 1);
}

// A fragments of step I: the wave's own pair and, on its share steps, the fifth pair.
template <int BITS, int NP, int W, int I, bool FAST>
__device__ __forceinline__ void deq_a(const PairCodes<BITS>& cur, const ShareCodes<BITS>& sh,
                                      uint32_t magic, f16x8& A, f16x8& A4) {
  constexpr int J = I >> 1, S = I & 1;
  A = wfrag<BITS, J, FAST>(cur.cw[S][J], cur.hw[S], magic, cur.zp, cur.sp);
  if constexpr (share_step<NP, W, I>())
    A4 = wfrag<BITS, J, FAST>(sh.cw[J & 1], sh.hw, magic, sh.zp, sh.sp);
}

// Step I of the software pipeline: the matrix-core steps of step I run while the A fragments of
// step I + 1 are dequantised and its B fragments read, each into the register of token tile tt
// as soon as step I's steps have taken it (one B set: the registers this frees keep the
// five-pair instance from spilling).  The instruction order inside a step is otherwise left to
// the compiler (measured: forcing one matrix-core step / one LDS read / a few vector ops in turn
// was 4-6% slower); the barrier at the end keeps steps from mixing.
template <int BITS, int NP, int NTT, int W, int I, bool FAST>
__device__ __forceinline__ void wide_step(const PairCodes<BITS>& cur, const ShareCodes<BITS>& sh,
                                          const char* xs, int bsw, uint32_t magic,
                                          const f16x8& Acur, f16x8& Anxt, f16x8& A4,
                                          f16x8 (&B)[NTT], f32x16 (&acc)[NTT], f32x16 (&accs)[NTT]) {
  constexpr bool SH = share_step<NP, W, I>();
  const f16x8 A4cur = A4;
  if constexpr (I + 1 < 8) deq_a<BITS, NP, W, I + 1, FAST>(cur, sh, magic, Anxt, A4);
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    acc[tt] = mfma32(Acur, B[tt], acc[tt]);
    if constexpr (SH) accs[tt] = mfma32(A4cur, B[tt], accs[tt]);
    if constexpr (I + 1 < 8) B[tt] = load_b1<I + 1>(xs, bsw, tt);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int BITS, int NP, int NTT, int W, bool FAST>
__device__ __forceinline__ void wide_loop(const Rsrcs& R, const KArgs& a, char* xbase,
                                          const int (&voff)[4], int bsw, int tok0, int pair,
                                          int spair, int ntiles, int wave, const LaneMap& m,
                                          uint32_t magic, PairCodes<BITS> cur,
                                          f32x16 (&acc)[NTT], f32x16 (&accs)[NTT]) {
  constexpr int BN = 32 * NTT;
  PairCodes<BITS> nxt;
  ShareCodes<BITS> sh{}, shn;
  if constexpr (NP == 5) load_share<BITS, W>(sh, R, a, m, spair, ntiles, 0);
  f16x8 A0, A1, A4, B[NTT];
  for (int kb = 0; kb < a.KB; ++kb) {
    // everything this wave issued has landed (its share of X(kb), the codes of block kb) ...
    wait_vmcnt<0>();
    // ... and so has everyone else's; everyone is also done reading the other buffer
    __syncthreads();
    const bool more = kb + 1 < a.KB;
    if (more) {
      load_x_lds<BN>(R, a, xbase + ((kb + 1) & 1) * (BN * 256), voff, tok0, kb + 1, wave);
      load_pair(nxt, R, a, m, pair, ntiles, kb + 1);
      if constexpr (NP == 5) load_share<BITS, W>(shn, R, a, m, spair, ntiles, kb + 1);
    }
    const char* xs = xbase + (kb & 1) * (BN * 256);
    load_b<NTT, 0>(xs, bsw, B);
    deq_a<BITS, NP, W, 0, FAST>(cur, sh, magic, A0, A4);
    wide_step<BITS, NP, NTT, W, 0, FAST>(cur, sh, xs, bsw, magic, A0, A1, A4, B, acc, accs);
    wide_step<BITS, NP, NTT, W, 1, FAST>(cur, sh, xs, bsw, magic, A1, A0, A4, B, acc, accs);
    wide_step<BITS, NP, NTT, W, 2, FAST>(cur, sh, xs, bsw, magic, A0, A1, A4, B, acc, accs);
    // (step 3 also prepares step 4; in a half-empty block that reads LDS and codes that exist
    // but are never used)
    wide_step<BITS, NP, NTT, W, 3, FAST>(cur, sh, xs, bsw, magic, A1, A0, A4, B, acc, accs);
    if (kb * 128 + 64 < a.K) {
      wide_step<BITS, NP, NTT, W, 4, FAST>(cur, sh, xs, bsw, magic, A0, A1, A4, B, acc, accs);
      wide_step<BITS, NP, NTT, W, 5, FAST>(cur, sh, xs, bsw, magic, A1, A0, A4, B, acc, accs);
      wide_step<BITS, NP, NTT, W, 6, FAST>(cur, sh, xs, bsw, magic, A0, A1, A4, B, acc, accs);
      wide_step<BITS, NP, NTT, W, 7, FAST>(cur, sh, xs, bsw, magic, A1, A0, A4, B, acc, accs);
    }
    if (more) {
      cur = nxt;
      if constexpr (NP == 5) sh = shn;
    }
  }
}

// The wave index selects the share steps at compile time (one copy of the loop per wave for
// five-pair workgroups, one copy in all for four).
template <int BITS, int NP, int NTT, bool FAST>
__device__ __forceinline__ void wide_loop_w(const Rsrcs& R, const KArgs& a, char* xbase,
                                            const int (&voff)[4], int bsw, int tok0, int pair,
                                            int spair, int ntiles, int wave, const LaneMap& m,
                                            uint32_t magic, const PairCodes<BITS>& cur,
                                            f32x16 (&acc)[NTT], f32x16 (&accs)[NTT]) {
#define W4_WIDE_LOOP(W)                                                                         \
  wide_loop<BITS, NP, NTT, W, FAST>(R, a, xbase, voff, bsw, tok0, pair, spair, ntiles, wave, m, \
                                    magic, cur, acc, accs)
  if constexpr (NP == 5) {
    switch (wave) {
      case 0: W4_WIDE_LOOP(0); break;
      case 1: W4_WIDE_LOOP(1); break;
      case 2: W4_WIDE_LOOP(2); break;
      default: W4_WIDE_LOOP(3); break;
    }
  } else {
    W4_WIDE_LOOP(0);
  }
#undef W4_WIDE_LOOP
}

template <int BITS, int NP, int NTT, int EPI, int OCC>
__global__ __launch_bounds__(256, OCC) void wide_kernel(KArgs a, int nrb, int ntb) {
  constexpr int BN = 32 * NTT;   // tokens per workgroup
  constexpr int TILES = 2 * NP;  // 16-row tiles per workgroup
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const xbase = smem;  // two buffers of BN x 256 bytes

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = a.rows / 16;

  // XCD-aware order: XCD x (= blockIdx % 8) takes a contiguous run of tiles, token-block major.
  const int G = nrb * ntb;
  const int b = blockIdx.x, xcd = b % kXCD, l = b / kXCD;
  const int q = G / kXCD, rem = G % kXCD;
  const int t_idx = xcd * q + min(xcd, rem) + l;
  const int rb = t_idx % nrb, tb = t_idx / nrb;
  const int tok0 = tb * BN;
  const int pair = rb * NP + wave, spair = rb * NP + 4;
  const uint32_t magic = vgpr_const(0x64006400u);
  const LaneMap m = lane_map(a, lane);

  Rsrcs R;
  R.x = rsrc(a.x, (uint32_t)((size_t)a.T * a.K * 2));
  R.w = rsrc(a.w, (uint32_t)((size_t)ntiles * a.KB * block_bytes(BITS)));
  R.s = rsrc(a.sc, (uint32_t)((size_t)ntiles * a.KB * 4 * a.szw));
  R.z = rsrc(a.zr, (uint32_t)((size_t)ntiles * a.KB * 4 * a.szw));
  int voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = lane >> 4;                      // row within the instruction
    const int chunk = (lane & 15) ^ (4 * i + rl);  // source chunk stored at this lane's slot
    voff[i] = (rl * a.K + chunk * 8) * 2;
  }
  const int brow = lane & 31;
  const int bsw = brow * 256 + 16 * ((4 * (lane >> 5)) ^ (brow & 15));

  f32x16 acc[NTT], accs[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    acc[tt] = f32x16{};
    accs[tt] = f32x16{};
  }

  load_x_lds<BN>(R, a, xbase, voff, tok0, 0, wave);
  PairCodes<BITS> cur;
  load_pair(cur, R, a, m, pair, ntiles, 0);

  // Are all zero-points of this workgroup's rows integers (1024 + z exact in fp16)?  One vote
  // for the whole kernel run of this workgroup, so the two main loops below are separate code
  // paths (a per-block branch would make the register allocator hold both at once).
  bool exact = true;
  {
    const int zbase = rb * TILES * a.KB * 4 * a.szw;  // bytes: zero-points of the row block
    const int zbytes = TILES * a.KB * 4 * a.szw;
    const f16x2 c1024 = {(f16)1024.0f, (f16)1024.0f};
    constexpr int STEP = 256 * 16;  // bytes per load instruction of the workgroup
    for (int off0 = threadIdx.x * 16; off0 < zbytes; off0 += 8 * STEP) {
      // eight loads in flight per pass (one pass up to K = 6144 with 160-row workgroups);
      // whole offset in the range-checked lane operand: rows past the last tile read zero
      u32x4 zz[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        zz[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.z, zbase + off0 + u * STEP, 0, 0));
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          exact = exact && (off0 + u * STEP >= zbytes ||
                            __builtin_bit_cast(uint32_t, (as_h2(zz[u][e]) + c1024) - c1024) == zz[u][e]);
    }
  }
  if (__syncthreads_and(exact))
    wide_loop_w<BITS, NP, NTT, true>(R, a, xbase, voff, bsw, tok0, pair, spair, ntiles, wave, m,
                                     magic, cur, acc, accs);
  else
    wide_loop_w<BITS, NP, NTT, false>(R, a, xbase, voff, bsw, tok0, pair, spair, ntiles, wave,
                                      m, magic, cur, acc, accs);

#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) store_pair<EPI>(a, acc[tt], pair, tok0 + 32 * tt, ntiles, lane);

  if constexpr (NP == 5) {
    // Fifth pair: wave w holds the partial sums of k-steps (j, w/2), j in {2 (w%2), 2 (w%2)+1}
    // of every block.  The four are added in wave order through LDS (the activation buffers
    // are free once every wave has left the loop); wave w finishes token tiles w, w + 4, ...
    static_assert(4 * NTT * 16 * 64 * 4 <= 2 * BN * 256, "reduction fits the activation buffers");
    float* red = reinterpret_cast<float*>(smem);
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((wave * NTT + tt) * 16 + v) * 64 + lane] = accs[tt][v];
    __syncthreads();
    for (int tt = wave; tt < NTT; tt += 4) {
      f32x16 sum;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float s = red[((0 * NTT + tt) * 16 + v) * 64 + lane];
        s += red[((1 * NTT + tt) * 16 + v) * 64 + lane];
        s += red[((2 * NTT + tt) * 16 + v) * 64 + lane];
        s += red[((3 * NTT + tt) * 16 + v) * 64 + lane];
        sum[v] = s;
      }
      store_pair<EPI>(a, sum, spair, tok0 + 32 * tt, ntiles, lane);
    }
  }
}

template <int BITS, int NP, int NTT, int EPI>
hipError_t run(const KArgs& a, hipStream_t stream) {
  constexpr int BN = 32 * NTT, TILES = 2 * NP;
  // two waves per SIMD (two workgroups per compute unit) when the tile's registers allow it
  constexpr int OCC = (NTT <= 4) ? 2 : 1;
  const int ntiles = a.rows / 16;
  const int nrb = (ntiles + TILES - 1) / TILES;
  const int ntb = (a.T + BN - 1) / BN;
  const size_t lds = (size_t)2 * BN * 256;
  return launch_kernel(&wide_kernel<BITS, NP, NTT, EPI, OCC>, dim3(nrb * ntb), dim3(256), lds,
                       stream, a, nrb, ntb);
}

template <int BITS, int EPI>
hipError_t pick(const KArgs& a, hipStream_t stream) {
  const int ntiles = a.rows / 16;
  // 160-row workgroups (5 pairs) divide the 5120-row projections into 32 row blocks; the
  // SwiGLU pair layout (gate, up) keeps every 32-row pair inside one output tile either way.
  const bool five = (ntiles % 10 == 0);
  // 128-token tiles, two workgroups per compute unit (measured against 256-token tiles with
  // one workgroup per compute unit: 290 vs 296 us at 5120 x 6144, T = 4096; the narrower tile
  // re-dequantises each weight block twice as often but lets two waves share each SIMD)
  if (five) return run<BITS, 5, 4, EPI>(a, stream);
  return run<BITS, 4, 4, EPI>(a, stream);
}

template <int BITS>
hipError_t pick_epi(int epi, const KArgs& a, hipStream_t stream) {
  if (epi == EPI_SWIGLU) return pick<BITS, EPI_SWIGLU>(a, stream);
  if (epi == EPI_ADD) return pick<BITS, EPI_ADD>(a, stream);
  return pick<BITS, EPI_STORE>(a, stream);
}

}  // namespace

hipError_t launch_wide(int bits, int epi, const KArgs& a, hipStream_t stream) {
  return bits == 5 ? pick_epi<5>(epi, a, stream) : pick_epi<4>(epi, a, stream);
}

}  // namespace w4
