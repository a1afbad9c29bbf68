// Wavefront GEMV path: exact T = 1..4 token columns (single-stream decode, MTP verify).
//
// Prior art: the SIMT split GEMVs of the ninfer-3080 performance notes ("Why the round cost
// too much": their cost grows with every column; the MMA kernel replaced them from T = 3).
//
// gfx950 design.  Same work split as the narrow path -- a workgroup owns RT 16-row tiles, its
// four waves stream four contiguous K ranges with one coalesced 16-byte load per lane per
// packed block -- but the products are packed-fp16 dot products (v_dot2_f32_f16) into fp32,
// one accumulator per (row tile, token), so nothing is padded to 16 tokens.  Lanes of a lane
// group hold disjoint k slots of the same row; they are combined with two cross-lane
// exchanges, then the four waves in LDS in a fixed order.
#include "device.h"
#include "kernels.h"

namespace w4 {
namespace {

using namespace w4dev;
using w4layout::block_bytes;

template <int BITS, int TT, int RT>
struct GemvTile {
  u32x4 cw[RT];
  uint32_t hw[RT];
  uint32_t sp[RT], zp[RT];
  u32x4 xv[TT][4];
};

template <int BITS, int TT, int RT>
__device__ __forceinline__ void gemv_load(GemvTile<BITS, TT, RT>& s, const KArgs& a, int tile0,
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
  const bool half_block = (kb * 128 + 64 >= a.K);
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const _Float16* xrow = a.x + (size_t)t * a.K + kb * 128 + 16 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = !(half_block && j >= 2);
      s.xv[t][j] = ok ? *reinterpret_cast<const u32x4*>(xrow + 64 * (j >> 1) + 8 * (j & 1))
                      : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int BITS, int TT, int RT, int J>
__device__ __forceinline__ void gemv_step(const GemvTile<BITS, TT, RT>& s, float (&acc)[RT][TT]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    f16x2 q[4];
    decode_q<BITS, J>(s.cw[rt][J], s.hw[rt], q);
    const f16x2 z2 = splat<(J >> 1)>(s.zp[rt]);
    const f16x2 s2 = splat<(J >> 1)>(s.sp[rt]);
    f16x2 wv[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) wv[p] = (q[p] - z2) * s2;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      float v = acc[rt][t];
#pragma unroll
      for (int p = 0; p < 4; ++p) v = __builtin_amdgcn_fdot2(wv[p], as_h2(s.xv[t][J][p]), v, false);
      acc[rt][t] = v;
    }
  }
}

template <int BITS, int TT, int RT, int EPI>
__global__ __launch_bounds__(256) void gemv_kernel(KArgs a) {
  __shared__ float red[4][RT][TT][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntiles = a.rows / 16;
  const int tile0 = blockIdx.x * RT;
  const int kb0 = (a.KB * wave) / 4, kb1 = (a.KB * (wave + 1)) / 4;

  float acc[RT][TT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[rt][t] = 0.f;

  if (kb0 < kb1) {
    GemvTile<BITS, TT, RT> cur, nxt;
    gemv_load(cur, a, tile0, ntiles, kb0, lane);
    for (int kb = kb0; kb < kb1; ++kb) {
      if (kb + 1 < kb1) gemv_load(nxt, a, tile0, ntiles, kb + 1, lane);
      gemv_step<BITS, TT, RT, 0>(cur, acc);
      gemv_step<BITS, TT, RT, 1>(cur, acc);
      gemv_step<BITS, TT, RT, 2>(cur, acc);
      gemv_step<BITS, TT, RT, 3>(cur, acc);
      cur = nxt;
    }
  }

  // Combine the four lane groups (same row, disjoint k) -- identical order in every lane.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      float v = acc[rt][t];
      v = v + __shfl_xor(v, 16);
      v = v + __shfl_xor(v, 32);
      acc[rt][t] = v;
    }
  if (lane < 16) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < TT; ++t) red[wave][rt][t][lane] = acc[rt][t];
  }
  __syncthreads();

  if constexpr (EPI == EPI_SWIGLU) {
    constexpr int ITEMS = (RT / 2) * TT * 16;
    for (int i = threadIdx.x; i < ITEMS; i += 256) {
      const int row = i & 15, t = (i >> 4) % TT, p = (i >> 4) / TT;
      const int gtile = tile0 + 2 * p;
      if (gtile >= ntiles) continue;
      const float gv = ((red[0][2 * p][t][row] + red[1][2 * p][t][row]) + red[2][2 * p][t][row]) +
                       red[3][2 * p][t][row];
      const float uv = ((red[0][2 * p + 1][t][row] + red[1][2 * p + 1][t][row]) +
                        red[2][2 * p + 1][t][row]) + red[3][2 * p + 1][t][row];
      store_one<EPI>(a.out, a.res, (size_t)t * a.ldo + (gtile >> 1) * 16 + row, gv, uv);
    }
  } else {
    constexpr int ITEMS = RT * TT * 16;
    for (int i = threadIdx.x; i < ITEMS; i += 256) {
      const int row = i & 15, t = (i >> 4) % TT, rt = (i >> 4) / TT;
      const int tile = tile0 + rt;
      if (tile >= ntiles) continue;
      const float v = ((red[0][rt][t][row] + red[1][rt][t][row]) + red[2][rt][t][row]) +
                      red[3][rt][t][row];
      store_one<EPI>(a.out, a.res, (size_t)t * a.ldo + tile * 16 + row, v, 0.f);
    }
  }
}

template <int BITS, int TT, int RT, int EPI>
hipError_t run(const KArgs& a, hipStream_t stream) {
  const int ntiles = a.rows / 16;
  const int grid = (ntiles + RT - 1) / RT;
  hipLaunchKernelGGL((gemv_kernel<BITS, TT, RT, EPI>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int BITS, int TT, int EPI>
hipError_t pick_rt(const KArgs& a, hipStream_t stream) {
  const int ntiles = a.rows / 16;
  if constexpr (EPI == EPI_SWIGLU) {
    return run<BITS, TT, 2, EPI>(a, stream);
  } else {
    if (ntiles >= 2 * 768) return run<BITS, TT, 2, EPI>(a, stream);
    return run<BITS, TT, 1, EPI>(a, stream);
  }
}

template <int BITS, int EPI>
hipError_t pick_t(const KArgs& a, hipStream_t stream) {
  switch (a.T) {
    case 1: return pick_rt<BITS, 1, EPI>(a, stream);
    case 2: return pick_rt<BITS, 2, EPI>(a, stream);
    case 3: return pick_rt<BITS, 3, EPI>(a, stream);
    default: return pick_rt<BITS, 4, EPI>(a, stream);
  }
}

template <int BITS>
hipError_t pick_epi(int epi, const KArgs& a, hipStream_t stream) {
  if (epi == EPI_SWIGLU) return pick_t<BITS, EPI_SWIGLU>(a, stream);
  if (epi == EPI_ADD) return pick_t<BITS, EPI_ADD>(a, stream);
  return pick_t<BITS, EPI_STORE>(a, stream);
}

}  // namespace

hipError_t launch_gemv(int bits, int epi, const KArgs& a, hipStream_t stream) {
  return bits == 5 ? pick_epi<5>(epi, a, stream) : pick_epi<4>(epi, a, stream);
}

}  // namespace w4
