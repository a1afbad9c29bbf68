// Narrow matrix-core path: T up to 16/32/64 token columns (batched decode, speculative verify).
//
// Prior art: the small-T MMA kernels of the ninfer-3080 performance notes ("What changed":
// permuted k order, activation slabs shared by several row tiles; "What is left at C1 / C8":
// the T=32 kernel is latency bound and the lever is operand movement and occupancy).
//
// gfx950 design.  A workgroup owns RT 16-row tiles and all T tokens (padded to NT*16).  Its
// four waves split K into four contiguous ranges, so every packed code is loaded exactly once
// chip-wide, straight into the lane that feeds it to the matrix core: the packed layout is the
// A-operand order, so dequantisation happens in registers with no LDS round trip.  Each wave
// loads the activation fragments for its K range once per k-block and reuses them across its
// RT row tiles.  The four partial sums are combined in LDS in a fixed order (deterministic),
// then the epilogue (store / SwiGLU / residual add) writes fp16 quads.
#include "device.h"
#include "kernels.h"

namespace w4 {
namespace {

using namespace w4dev;
using w4layout::block_bytes;

template <int BITS, int NT, int RT>
struct NarrowTile {
  u32x4 cw[RT];
  uint32_t hw[RT];
  uint32_t sp[RT], zp[RT];
  u32x4 xb[NT][4];
};

template <int BITS, int NT, int RT>
__device__ __forceinline__ void narrow_load(NarrowTile<BITS, NT, RT>& s, const KArgs& a, int tile0,
                                            int ntiles, int kb, int lane) {
  constexpr int BLK = block_bytes(BITS);
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int tile = min(tile0 + rt, ntiles - 1);
    const size_t boff = ((size_t)tile * a.KB + kb) * BLK;
    s.cw[rt] = *reinterpret_cast<const u32x4*>(a.w + boff + lane * 16);
    if constexpr (BITS == 5) s.hw[rt] = *reinterpret_cast<const uint32_t*>(a.w + boff + 1024 + lane * 4);
    else s.hw[rt] = 0;
    const size_t soff = ((size_t)tile * a.KB + kb) * 16 + r;
    s.sp[rt] = a.sc[soff];
    s.zp[rt] = a.zr[soff];
  }
  const bool half_block = (kb * 128 + 64 >= a.K);  // second group of this block is padding
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int t = tt * 16 + r;
    const _Float16* xrow = a.x + (size_t)t * a.K + kb * 128 + 16 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = (t < a.T) && !(half_block && j >= 2);
      s.xb[tt][j] = ok ? *reinterpret_cast<const u32x4*>(xrow + 64 * (j >> 1) + 8 * (j & 1))
                       : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int BITS, int NT, int RT, int J>
__device__ __forceinline__ void narrow_step(const NarrowTile<BITS, NT, RT>& s, f32x4 (&acc)[RT][NT]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const f16x8 A = dequant8<BITS, J>(s.cw[rt][J], s.hw[rt], splat<(J >> 1)>(s.zp[rt]),
                                      splat<(J >> 1)>(s.sp[rt]));
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      acc[rt][tt] = mfma16(A, __builtin_bit_cast(f16x8, s.xb[tt][J]), acc[rt][tt]);
  }
}

template <int BITS, int NT, int RT, int EPI>
__global__ __launch_bounds__(256) void narrow_kernel(KArgs a) {
  __shared__ f32x4 red[4][RT][NT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntiles = a.rows / 16;
  const int tile0 = blockIdx.x * RT;
  const int kb0 = (a.KB * wave) / 4, kb1 = (a.KB * (wave + 1)) / 4;

  f32x4 acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (kb0 < kb1) {
    NarrowTile<BITS, NT, RT> cur, nxt;
    narrow_load(cur, a, tile0, ntiles, kb0, lane);
    for (int kb = kb0; kb < kb1; ++kb) {
      if (kb + 1 < kb1) narrow_load(nxt, a, tile0, ntiles, kb + 1, lane);
      narrow_step<BITS, NT, RT, 0>(cur, acc);
      narrow_step<BITS, NT, RT, 1>(cur, acc);
      narrow_step<BITS, NT, RT, 2>(cur, acc);
      narrow_step<BITS, NT, RT, 3>(cur, acc);
      cur = nxt;
    }
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) red[wave][rt][tt][lane] = acc[rt][tt];
  __syncthreads();

  if constexpr (EPI == EPI_SWIGLU) {
    constexpr int ITEMS = (RT / 2) * NT * 64;
    for (int i = threadIdx.x; i < ITEMS; i += 256) {
      const int l = i & 63, tt = (i >> 6) % NT, p = (i >> 6) / NT;
      const int gtile = tile0 + 2 * p;
      if (gtile >= ntiles) continue;
      const int t = tt * 16 + (l & 15);
      if (t >= a.T) continue;
      const f32x4 gv = ((red[0][2 * p][tt][l] + red[1][2 * p][tt][l]) + red[2][2 * p][tt][l]) +
                       red[3][2 * p][tt][l];
      const f32x4 uv = ((red[0][2 * p + 1][tt][l] + red[1][2 * p + 1][tt][l]) +
                        red[2][2 * p + 1][tt][l]) + red[3][2 * p + 1][tt][l];
      const int n = (gtile >> 1) * 16 + 4 * (l >> 4);
      store_quad<EPI>(a.out, a.res, (size_t)t * a.ldo + n, gv, uv);
    }
  } else {
    constexpr int ITEMS = RT * NT * 64;
    for (int i = threadIdx.x; i < ITEMS; i += 256) {
      const int l = i & 63, tt = (i >> 6) % NT, rt = (i >> 6) / NT;
      const int tile = tile0 + rt;
      if (tile >= ntiles) continue;
      const int t = tt * 16 + (l & 15);
      if (t >= a.T) continue;
      const f32x4 v = ((red[0][rt][tt][l] + red[1][rt][tt][l]) + red[2][rt][tt][l]) +
                      red[3][rt][tt][l];
      const int n = tile * 16 + 4 * (l >> 4);
      store_quad<EPI>(a.out, a.res, (size_t)t * a.ldo + n, v, f32x4{});
    }
  }
}

template <int BITS, int NT, int RT, int EPI>
hipError_t run(const KArgs& a, hipStream_t stream) {
  const int ntiles = a.rows / 16;
  const int grid = (ntiles + RT - 1) / RT;
  hipLaunchKernelGGL((narrow_kernel<BITS, NT, RT, EPI>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int BITS, int NT, int EPI>
hipError_t pick_rt(const KArgs& a, hipStream_t stream) {
  const int ntiles = a.rows / 16;
  if constexpr (EPI == EPI_SWIGLU) {
    return run<BITS, NT, 2, EPI>(a, stream);
  } else {
    // Keep at least ~3 workgroups per compute unit before sharing activations over 2 tiles.
    if (ntiles >= 2 * 768) return run<BITS, NT, 2, EPI>(a, stream);
    return run<BITS, NT, 1, EPI>(a, stream);
  }
}

template <int BITS, int EPI>
hipError_t pick_nt(int tn, const KArgs& a, hipStream_t stream) {
  if (tn <= 16) return pick_rt<BITS, 1, EPI>(a, stream);
  if (tn <= 32) return pick_rt<BITS, 2, EPI>(a, stream);
  return pick_rt<BITS, 4, EPI>(a, stream);
}

template <int BITS>
hipError_t pick_epi(int tn, int epi, const KArgs& a, hipStream_t stream) {
  if (epi == EPI_SWIGLU) return pick_nt<BITS, EPI_SWIGLU>(tn, a, stream);
  if (epi == EPI_ADD) return pick_nt<BITS, EPI_ADD>(tn, a, stream);
  return pick_nt<BITS, EPI_STORE>(tn, a, stream);
}

}  // namespace

hipError_t launch_narrow(int tn, int bits, int epi, const KArgs& a, hipStream_t stream) {
  return bits == 5 ? pick_epi<5>(tn, epi, a, stream) : pick_epi<4>(tn, epi, a, stream);
}

}  // namespace w4
