// Wide matrix-core path: prefill widths (hundreds to thousands of token columns).
//
// Prior art: the prefill schedules of the ninfer-3080 performance notes ("The token tile, and
// why it was hiding": a token tile of BN columns re-streams the whole weight matrix T/BN
// times, so the tile must be wide; "What is still missing": the lever is the mainloop --
// double buffering and a conflict-free shared layout).
//
// gfx950 design.  A workgroup of four waves (2 x 2) owns BM = 32*RTW rows and BN = 32*NTW
// tokens.  The activation tile X[BN][128] of each k-block is staged in LDS (rows padded by
// 16 bytes so a 16-lane read phase touches 64 distinct banks) with a register double buffer:
// the next block's activations and codes are loaded from HBM while the matrix cores work on
// the current one.  Weights never touch LDS: each lane loads its packed codes in A-operand
// order and dequantises them in registers, and every dequantised fragment feeds NTW matrix
// core steps.  Each wave owns its outputs, so the epilogue writes straight from registers.
#include "device.h"
#include "kernels.h"

namespace w4 {
namespace {

using namespace w4dev;
using w4layout::block_bytes;

constexpr int LDX = 128 + 8;  // fp16 per staged activation row (16 B pad)

template <int BITS, int RTW>
struct WideCodes {
  u32x4 cw[RTW];
  uint32_t hw[RTW];
  uint32_t sp[RTW], zp[RTW];
};

template <int BITS, int RTW>
__device__ __forceinline__ void wide_load_codes(WideCodes<BITS, RTW>& c, const KArgs& a,
                                                int tile_base, int ntiles, int kb, int lane) {
  constexpr int BLK = block_bytes(BITS);
  const int r = lane & 15;
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int tile = min(tile_base + rt, ntiles - 1);
    const size_t boff = ((size_t)tile * a.KB + kb) * BLK;
    c.cw[rt] = *reinterpret_cast<const u32x4*>(a.w + boff + lane * 16);
    if constexpr (BITS == 5) c.hw[rt] = *reinterpret_cast<const uint32_t*>(a.w + boff + 1024 + lane * 4);
    else c.hw[rt] = 0;
    const size_t soff = ((size_t)tile * a.KB + kb) * 16 + r;
    c.sp[rt] = a.sc[soff];
    c.zp[rt] = a.zr[soff];
  }
}

template <int BN>
__device__ __forceinline__ void wide_load_x(u32x4 (&xr)[BN / 16], const KArgs& a, int tok0, int kb) {
#pragma unroll
  for (int c = 0; c < BN / 16; ++c) {
    const int idx = threadIdx.x + 256 * c;
    const int tok = idx >> 4, kc = idx & 15;
    const int t = tok0 + tok, k = kb * 128 + kc * 8;
    xr[c] = (t < a.T && k < a.K) ? *reinterpret_cast<const u32x4*>(a.x + (size_t)t * a.K + k)
                                 : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int BN>
__device__ __forceinline__ void wide_store_x(const u32x4 (&xr)[BN / 16], _Float16* xs) {
#pragma unroll
  for (int c = 0; c < BN / 16; ++c) {
    const int idx = threadIdx.x + 256 * c;
    const int tok = idx >> 4, kc = idx & 15;
    *reinterpret_cast<u32x4*>(xs + tok * LDX + kc * 8) = xr[c];
  }
}

template <int BITS, int RTW, int NTW, int J>
__device__ __forceinline__ void wide_step(const WideCodes<BITS, RTW>& c, const _Float16* xs,
                                          int tokw, int lane, f32x4 (&acc)[RTW][NTW]) {
  const int r = lane & 15, g = lane >> 4;
  f16x8 b[NTW];
#pragma unroll
  for (int tt = 0; tt < NTW; ++tt)
    b[tt] = *reinterpret_cast<const f16x8*>(xs + (tokw + tt * 16 + r) * LDX + 64 * (J >> 1) +
                                            16 * g + 8 * (J & 1));
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const f16x8 A = dequant8<BITS, J>(c.cw[rt][J], c.hw[rt], splat<(J >> 1)>(c.zp[rt]),
                                      splat<(J >> 1)>(c.sp[rt]));
#pragma unroll
    for (int tt = 0; tt < NTW; ++tt) acc[rt][tt] = mfma16(A, b[tt], acc[rt][tt]);
  }
}

template <int BITS, int RTW, int NTW, int EPI>
__global__ __launch_bounds__(256) void wide_kernel(KArgs a) {
  constexpr int BN = 32 * NTW;       // tokens per workgroup
  constexpr int TILES = 2 * RTW;     // row tiles per workgroup
  __shared__ _Float16 xs[2][BN * LDX];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave & 1, wt = wave >> 1;
  const int ntiles = a.rows / 16;
  const int nrb = (ntiles + TILES - 1) / TILES;
  const int rb = blockIdx.x % nrb, tb = blockIdx.x / nrb;
  const int tok0 = tb * BN;
  const int tile_base = rb * TILES + wr * RTW;
  const int tokw = wt * NTW * 16;  // this wave's first token inside the tile

  f32x4 acc[RTW][NTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int tt = 0; tt < NTW; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 xr[BN / 16];
  wide_load_x<BN>(xr, a, tok0, 0);
  WideCodes<BITS, RTW> cur, nxt;
  wide_load_codes(cur, a, tile_base, ntiles, 0, lane);
  wide_store_x<BN>(xr, xs[0]);
  __syncthreads();

  for (int kb = 0; kb < a.KB; ++kb) {
    const _Float16* xcur = xs[kb & 1];
    const bool more = kb + 1 < a.KB;
    if (more) {
      wide_load_x<BN>(xr, a, tok0, kb + 1);
      wide_load_codes(nxt, a, tile_base, ntiles, kb + 1, lane);
    }
    wide_step<BITS, RTW, NTW, 0>(cur, xcur, tokw, lane, acc);
    wide_step<BITS, RTW, NTW, 1>(cur, xcur, tokw, lane, acc);
    wide_step<BITS, RTW, NTW, 2>(cur, xcur, tokw, lane, acc);
    wide_step<BITS, RTW, NTW, 3>(cur, xcur, tokw, lane, acc);
    if (more) wide_store_x<BN>(xr, xs[(kb + 1) & 1]);
    __syncthreads();
    cur = nxt;
  }

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
  hipLaunchKernelGGL((wide_kernel<BITS, RTW, NTW, EPI>), dim3(nrb * ntb), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int BITS, int EPI>
hipError_t pick(const KArgs& a, hipStream_t stream) {
  if constexpr (EPI == EPI_SWIGLU) {
    return run<BITS, 4, 4, EPI>(a, stream);
  } else {
    const int ntiles = a.rows / 16;
    // 160-row tiles divide the 5120-row projections into 32 row blocks.
    if (ntiles % 10 == 0) return run<BITS, 5, 4, EPI>(a, stream);
    return run<BITS, 4, 4, EPI>(a, stream);
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
