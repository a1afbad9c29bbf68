// Wide matrix-core path: prefill widths (hundreds to thousands of token columns).
//
// Prior art: the prefill schedules of the ninfer-3080 performance notes ("The token tile, and
// why it was hiding": a token tile of BN columns re-streams the whole weight matrix T/BN times,
// so the tile must be wide; a grid swizzle for cache reuse bought nothing there because the
// passes themselves had to go; "What is still missing": the mainloop -- double buffering and a
// conflict-free shared layout).
//
// gfx950 design.
//  * Workgroup = 4 waves in a 2 x 2 arrangement; a wave owns RTW 16-row tiles x NTW 16-token
//    tiles (80 x 128 for 5120-row projections), so every dequantised weight fragment feeds NTW
//    matrix-core steps and the dequantisation (13-19 vector ops per packed word) stays below
//    the matrix-core time of the same block.
//  * Weights never touch LDS: the packed layout is the A-operand order, each lane loads its
//    codes with one 16-byte load per 16-row tile and k-block and dequantises in registers.
//  * The activation tile X[BN tokens][128 columns] of each k-block is loaded straight into LDS
//    with global_load_lds_dwordx4 (no register staging), double buffered, one barrier per
//    k-block.  16-byte chunks are stored XOR-swizzled by token row (chunk c of row r sits at
//    c ^ (r & 15)), so the 16 lanes of a read phase hit 16 distinct bank groups.
//  * Tiles are ordered so that the workgroups running at the same time on one XCD (round-robin
//    dispatch) cover all row blocks of the same token block: that activation tile is fetched
//    into the XCD's L2 once and shared, instead of being re-read per row block.
//  * Integer zero-points (checked exactly and wave-uniformly per block) take a 13-op (4-bit) /
//    19-op (5-bit) dequantisation; fractional ones the general form.
#include "device.h"
#include "kernels.h"

namespace w4 {
namespace {

using namespace w4dev;
using w4layout::block_bytes;

constexpr int kXCD = 8;  // gfx950 (MI350 series): 8 accelerator complex dies, round-robin dispatch

__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// Wait until at most n vector-memory operations of this wave are outstanding (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// (a & mask) | c in one v_and_or_b32 (the compiler otherwise forms and + and + or3)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(c));
  return r;
}

template <int BITS, int J>
__device__ __forceinline__ void wbiased(uint32_t w, uint32_t hiw, uint32_t magic, uint32_t u[4]) {
  const uint32_t w8 = w >> 8;
  u[0] = (w & 0x000F000Fu) | magic;
  u[1] = (w & 0x00F000F0u) | magic;
  u[2] = (w8 & 0x000F000Fu) | magic;
  u[3] = (w8 & 0x00F000F0u) | magic;
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

template <int BITS, int J, bool FAST>
__device__ __forceinline__ f16x8 wfrag(uint32_t w, uint32_t hiw, uint32_t magic, f16x2 z2, f16x2 b0,
                                       f16x2 b1, f16x2 s2) {
  uint32_t u[4];
  wbiased<BITS, J>(w, hiw, magic, u);
  const f16x2 c16th = {(f16)0.0625f, (f16)0.0625f};
  if constexpr (FAST) {
    return cat8((as_h2(u[0]) + b0) * s2, (as_h2(u[1]) * c16th + b1) * s2, (as_h2(u[2]) + b0) * s2,
                (as_h2(u[3]) * c16th + b1) * s2);
  } else {
    const f16x2 c1024 = {(f16)1024.0f, (f16)1024.0f}, c64 = {(f16)64.0f, (f16)64.0f};
    return cat8(((as_h2(u[0]) - c1024) - z2) * s2, ((as_h2(u[1]) * c16th - c64) - z2) * s2,
                ((as_h2(u[2]) - c1024) - z2) * s2, ((as_h2(u[3]) * c16th - c64) - z2) * s2);
  }
}

template <int BITS, int RTW>
struct Codes {
  u32x4 cw[RTW];
  uint32_t hw[RTW], sp[RTW], zp[RTW];
};

// Buffer resource over `bytes` bytes at `base` (gfx9 raw buffer, 32-bit offsets; reads past
// the end return zero instead of faulting).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

struct Rsrcs {
  __amdgpu_buffer_rsrc_t x, w, s, z;
};

template <int BITS, int RTW>
__device__ __forceinline__ void load_codes(Codes<BITS, RTW>& c, const Rsrcs& R, const KArgs& a,
                                           int tile_base, int ntiles, int kb, int lane) {
  constexpr int BLK = block_bytes(BITS);
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int tile = min(tile_base + rt, ntiles - 1);
    const int bi = tile * a.KB + kb;
    c.cw[rt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.w, lane * 16, bi * BLK, 0));
    if constexpr (BITS == 5) c.hw[rt] = __builtin_amdgcn_raw_buffer_load_b32(R.w, 1024 + lane * 4, bi * BLK, 0);
    else c.hw[rt] = 0;
    c.sp[rt] = __builtin_amdgcn_raw_buffer_load_b32(R.s, (lane & 15) * 4, bi * 64, 0);
    c.zp[rt] = __builtin_amdgcn_raw_buffer_load_b32(R.z, (lane & 15) * 4, bi * 64, 0);
  }
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
__device__ __forceinline__ void load_x_lds(const Rsrcs& R, const KArgs& a, _Float16* xs,
                                           const int (&voff)[4], int tok0, int kb, int wave) {
  constexpr int PER_WAVE = BN / 16;  // instructions per wave
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int r0 = (wave * PER_WAVE + i) * 4;
    const int rowoff = ((tok0 + r0) * a.K + kb * 128) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        R.x, (__attribute__((address_space(3))) void*)(xs + r0 * 128), 16,
        voff[(r0 & 15) >> 2] + rowoff, 0, 0, 0);
  }
}

template <int BITS, int RTW, int NTW, int J, bool FAST>
__device__ __forceinline__ void wide_j(const Codes<BITS, RTW>& c, const _Float16* xs, int tokw,
                                       int lane, uint32_t magic, const f16x2* nb0, const f16x2* nb1,
                                       f32x4 (&acc)[RTW][NTW]) {
  const int r = lane & 15, g = lane >> 4;
  constexpr int cj = 8 * (J >> 1) + (J & 1);
  f16x8 b[NTW];
#pragma unroll
  for (int tt = 0; tt < NTW; ++tt) {
    const int row = tokw + tt * 16 + r;
    b[tt] = *reinterpret_cast<const f16x8*>(xs + row * 128 + (((cj + 2 * g) ^ r) * 8));
  }
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const f16x8 A = wfrag<BITS, J, FAST>(c.cw[rt][J], c.hw[rt], magic, splat<(J >> 1)>(c.zp[rt]),
                                         splat<(J >> 1)>(__builtin_bit_cast(uint32_t, nb0[rt])),
                                         splat<(J >> 1)>(__builtin_bit_cast(uint32_t, nb1[rt])),
                                         splat<(J >> 1)>(c.sp[rt]));
#pragma unroll
    for (int tt = 0; tt < NTW; ++tt) acc[rt][tt] = mfma16(A, b[tt], acc[rt][tt]);
  }
  // keep the scheduler from hoisting the next step's fragments over these matrix-core steps
  // (that would hold four steps of B fragments live and spill)
  __builtin_amdgcn_sched_barrier(0);
}

template <int BITS, int RTW, int NTW, bool FAST>
__device__ __forceinline__ void wide_block(const Codes<BITS, RTW>& c, const _Float16* xs, int tokw,
                                           int lane, uint32_t magic, bool half_block,
                                           f32x4 (&acc)[RTW][NTW]) {
  f16x2 nb0[RTW], nb1[RTW];
  const f16x2 c1024 = {(f16)1024.0f, (f16)1024.0f}, c64 = {(f16)64.0f, (f16)64.0f};
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    nb0[rt] = -(as_h2(c.zp[rt]) + c1024);
    nb1[rt] = -(as_h2(c.zp[rt]) + c64);
  }
  wide_j<BITS, RTW, NTW, 0, FAST>(c, xs, tokw, lane, magic, nb0, nb1, acc);
  wide_j<BITS, RTW, NTW, 1, FAST>(c, xs, tokw, lane, magic, nb0, nb1, acc);
  if (!half_block) {
    wide_j<BITS, RTW, NTW, 2, FAST>(c, xs, tokw, lane, magic, nb0, nb1, acc);
    wide_j<BITS, RTW, NTW, 3, FAST>(c, xs, tokw, lane, magic, nb0, nb1, acc);
  }
}

template <int BITS, int RTW, int NTW, int BN, bool FAST>
__device__ __forceinline__ void wide_loop(const Rsrcs& R, const KArgs& a, _Float16* xbase,
                                          const int (&voff)[4], int tok0, int tile_base, int ntiles,
                                          int tokw, int wave, int lane, uint32_t magic,
                                          Codes<BITS, RTW> cur, f32x4 (&acc)[RTW][NTW]) {
  Codes<BITS, RTW> nxt;
  for (int kb = 0; kb < a.KB; ++kb) {
    // everything this wave issued has landed: its share of X(kb) and the codes of block kb
    // (both are needed now; waiting for all keeps this independent of the load order) ...
    wait_vmcnt<0>();
    // ... and so has everyone else's; everyone is also done reading the other buffer
    __syncthreads();
    const bool more = kb + 1 < a.KB;
    if (more) {
      load_x_lds<BN>(R, a, xbase + ((kb + 1) & 1) * (BN * 128), voff, tok0, kb + 1, wave);
      load_codes(nxt, R, a, tile_base, ntiles, kb + 1, lane);
    }
    const _Float16* xs = xbase + (kb & 1) * (BN * 128);
    wide_block<BITS, RTW, NTW, FAST>(cur, xs, tokw, lane, magic, kb * 128 + 64 >= a.K, acc);
    if (more) cur = nxt;
  }
}

template <int BITS, int RTW, int NTW, int EPI>
__global__ __launch_bounds__(256, 1) void wide_kernel(KArgs a, int nrb, int ntb) {
  constexpr int BN = 32 * NTW;    // tokens per workgroup
  constexpr int TILES = 2 * RTW;  // row tiles per workgroup
  extern __shared__ __attribute__((aligned(16))) char smem[];
  _Float16* const xbase = reinterpret_cast<_Float16*>(smem);  // two buffers of BN x 128 fp16

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave & 1, wt = wave >> 1;
  const int ntiles = a.rows / 16;

  // XCD-aware order: XCD x (= blockIdx % 8) takes a contiguous run of tiles, token-block major.
  const int G = nrb * ntb;
  const int b = blockIdx.x, xcd = b % kXCD, l = b / kXCD;
  const int q = G / kXCD, rem = G % kXCD;
  const int t_idx = xcd * q + min(xcd, rem) + l;
  const int rb = t_idx % nrb, tb = t_idx / nrb;
  const int tok0 = tb * BN;
  const int tile_base = rb * TILES + wr * RTW;
  const int tokw = wt * NTW * 16;
  const uint32_t magic = vgpr_const(0x64006400u);

  Rsrcs R;
  R.x = rsrc(a.x, (uint32_t)((size_t)a.T * a.K * 2));
  R.w = rsrc(a.w, (uint32_t)((size_t)ntiles * a.KB * block_bytes(BITS)));
  R.s = rsrc(a.sc, (uint32_t)((size_t)ntiles * a.KB * 64));
  R.z = rsrc(a.zr, (uint32_t)((size_t)ntiles * a.KB * 64));
  int voff[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int rl = lane >> 4;                          // row within the instruction
    const int chunk = (lane & 15) ^ (4 * m + rl);      // source chunk stored at this lane's slot
    voff[m] = (rl * a.K + chunk * 8) * 2;
  }

  f32x4 acc[RTW][NTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int tt = 0; tt < NTW; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_x_lds<BN>(R, a, xbase, voff, tok0, 0, wave);
  Codes<BITS, RTW> cur;
  load_codes(cur, R, a, tile_base, ntiles, 0, lane);

  // Are all zero-points of this workgroup's rows integers (1024 + z exact in fp16)?  One vote
  // for the whole kernel run of this workgroup, so the two main loops below are separate code
  // paths (a per-block branch would make the register allocator hold both at once).
  bool exact = true;
  {
    const int zbase = rb * TILES * a.KB * 64;  // bytes: zero-points of the row block
    const int zbytes = TILES * a.KB * 64;
    const f16x2 c1024 = {(f16)1024.0f, (f16)1024.0f};
    for (int off = threadIdx.x * 16; off < zbytes; off += 256 * 16) {
      // whole offset in the range-checked lane operand: rows past the last tile read zero
      const u32x4 zz = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.z, zbase + off, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        exact = exact && (__builtin_bit_cast(uint32_t, (as_h2(zz[e]) + c1024) - c1024) == zz[e]);
    }
  }
  if (__syncthreads_and(exact))
    wide_loop<BITS, RTW, NTW, BN, true>(R, a, xbase, voff, tok0, tile_base, ntiles, tokw, wave,
                                        lane, magic, cur, acc);
  else
    wide_loop<BITS, RTW, NTW, BN, false>(R, a, xbase, voff, tok0, tile_base, ntiles, tokw, wave,
                                         lane, magic, cur, acc);

  const int r = lane & 15, quad = 4 * (lane >> 4);
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int p = 0; p < RTW / 2; ++p) {
      const int gtile = tile_base + 2 * p;
      if (gtile >= ntiles) continue;
#pragma unroll
      for (int tt = 0; tt < NTW; ++tt) {
        const int t = tok0 + tokw + tt * 16 + r;
        if (t < a.T)
          store_quad<EPI>(a.out, a.res, (size_t)t * a.ldo + (gtile >> 1) * 16 + quad,
                          acc[2 * p][tt], acc[2 * p + 1][tt]);
      }
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int tile = tile_base + rt;
      if (tile >= ntiles) continue;
#pragma unroll
      for (int tt = 0; tt < NTW; ++tt) {
        const int t = tok0 + tokw + tt * 16 + r;
        if (t < a.T)
          store_quad<EPI>(a.out, a.res, (size_t)t * a.ldo + tile * 16 + quad, acc[rt][tt],
                          f32x4{});
      }
    }
  }
}

template <int BITS, int RTW, int NTW, int EPI>
hipError_t run(const KArgs& a, hipStream_t stream) {
  constexpr int BN = 32 * NTW, TILES = 2 * RTW;
  const int ntiles = a.rows / 16;
  const int nrb = (ntiles + TILES - 1) / TILES;
  const int ntb = (a.T + BN - 1) / BN;
  const size_t lds = (size_t)2 * BN * 128 * sizeof(_Float16);
  hipLaunchKernelGGL((wide_kernel<BITS, RTW, NTW, EPI>), dim3(nrb * ntb), dim3(256), lds, stream,
                     a, nrb, ntb);
  return hipGetLastError();
}

template <int BITS, int EPI>
hipError_t pick(const KArgs& a, hipStream_t stream) {
  if constexpr (EPI == EPI_SWIGLU) {
    return run<BITS, 4, 8, EPI>(a, stream);
  } else {
    const int ntiles = a.rows / 16;
    // 160-row tiles divide the 5120-row projections into 32 row blocks.
    if (ntiles % 10 == 0) {
      // keep at least one workgroup per compute unit: narrower token tile for short prefill
      const long wg_wide = (long)(ntiles / 10) * ((a.T + 255) / 256);
      if (wg_wide >= 256) return run<BITS, 5, 8, EPI>(a, stream);
      return run<BITS, 5, 4, EPI>(a, stream);
    }
    return run<BITS, 4, 8, EPI>(a, stream);
  }
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
