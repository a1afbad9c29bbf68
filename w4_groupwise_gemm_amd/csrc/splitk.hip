// Split-K streaming matrix-core path for 17-32 token columns.
//
// Prior art: the small-T MMA kernels of the ninfer-3080 performance notes ("What is left at
// C8": the T=32 kernel is latency bound; the lever is operand movement and occupancy, a tile
// that puts more work in flight).
//
// gfx950 design.  At these widths the matrix-core work per weight byte is small and the
// dequantisation (13 vector ops per packed dword) dominates the compute, so the kernel is built
// for independent waves rather than lock-step ones:
//  * a workgroup of NW waves owns NP 32-row tile pairs and all (up to 32) tokens; the waves
//    split K into NW contiguous block ranges, so every code byte is loaded once, into the lane
//    that multiplies it, and no barrier is needed until the final reduction -- two waves per
//    SIMD overlap one's vector work with the other's matrix-core work and loads;
//  * each wave keeps D blocks of loads in flight: per pair the two 16-byte code slots of its
//    lanes (sets 0 and 1, the A-operand order of v_mfma_f32_32x32x16_f16 for a 32-row pair)
//    plus scale and zero-point words, and per block the activation fragments of its K range
//    (each lane's 32 contiguous k of a group are one 64-byte run of an activation row);
//    codes and activations of a block share one lead, so the in-order load counter never
//    waits for a later block;
//  * token rows beyond T read as zero (range-checked buffer loads) and are never stored;
//  * the NW partial sums are added in LDS in a fixed order (bitwise reproducible), then the
//    epilogue (store / SwiGLU / residual add) writes fp16 quads.
#include "device.h"
#include "kernels.h"
#include "tile32.h"

namespace w4 {
namespace {

using namespace w4dev;
using namespace t32;
using w4layout::block_bytes;

// Loads of one block for one wave.
template <int NP>
struct Blk {
  u32x4 cw[NP][2];  // code slots of sets 0 and 1
  uint32_t hw[NP][2];
  uint32_t sp[NP], zp[NP];
  u32x4 xb[8];  // activation fragment of step i = 2 J + S
};

template <int BITS, int NP>
__device__ __forceinline__ void issue(Blk<NP>& b, const Rsrcs& R, const KArgs& a, const LaneMap& m,
                                      int pair0, int ntiles, int kb, int xoff) {
  constexpr int BLK = block_bytes(BITS);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int tile = min(2 * (pair0 + p) + m.th, ntiles - 1);
    const int bi = tile * a.KB + kb;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      b.cw[p][s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.w, bi * BLK + m.slot16[s], 0, 0));
      b.hw[p][s] = BITS == 5 ? __builtin_amdgcn_raw_buffer_load_b32(R.w, bi * BLK + 1024 + m.slot16[s] / 4, 0, 0) : 0u;
    }
    b.sp[p] = __builtin_amdgcn_raw_buffer_load_b32(R.s, bi * 4 * a.szw + m.szoff, 0, 0);
    b.zp[p] = __builtin_amdgcn_raw_buffer_load_b32(R.z, bi * 4 * a.szw + m.szoff, 0, 0);
  }
  // step i = 2 J + S covers k = 64 (J / 2) + 16 (S + 2 h) + 8 (J % 2) + 0..7 of the block
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int J = i >> 1, S = i & 1;
    const int k = 64 * (J >> 1) + 16 * S + 8 * (J & 1);
    b.xb[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.x, xoff + (kb * 128 + k) * 2, 0, 0));
  }
}

template <int BITS, int NP, bool FAST>
__device__ __forceinline__ void block_math(const Blk<NP>& b, uint32_t magic, bool half,
                                           f32x16 (&acc)[NP]) {
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    if (J >= 2 && half) break;  // second group of a half-empty last block
#pragma unroll
    for (int S = 0; S < 2; ++S) {
      const f16x8 B = __builtin_bit_cast(f16x8, b.xb[2 * J + S]);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        f16x8 A;
        if (J == 0) A = wfrag<BITS, 0, FAST>(b.cw[p][S][0], b.hw[p][S], magic, b.zp[p], b.sp[p]);
        if (J == 1) A = wfrag<BITS, 1, FAST>(b.cw[p][S][1], b.hw[p][S], magic, b.zp[p], b.sp[p]);
        if (J == 2) A = wfrag<BITS, 2, FAST>(b.cw[p][S][2], b.hw[p][S], magic, b.zp[p], b.sp[p]);
        if (J == 3) A = wfrag<BITS, 3, FAST>(b.cw[p][S][3], b.hw[p][S], magic, b.zp[p], b.sp[p]);
        acc[p] = mfma32(A, B, acc[p]);
      }
    }
  }
}

template <int BITS, int NP, int NW, int D, int EPI>
__global__ __launch_bounds__(NW * 64) void splitk_kernel(KArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = a.rows / 16;
  const int pair0 = blockIdx.x * NP;
  const int KB = a.KB;
  const int kb0 = (KB * wave) / NW, kb1 = (KB * (wave + 1)) / NW;
  const bool half_last = (KB * 128 != a.K);
  const uint32_t magic = vgpr_const(0x64006400u);
  const LaneMap m = lane_map(a, lane);

  Rsrcs R;
  R.x = rsrc(a.x, (uint32_t)((size_t)a.T * a.K * 2));
  R.w = rsrc(a.w, (uint32_t)((size_t)ntiles * KB * block_bytes(BITS)));
  R.s = rsrc(a.sc, (uint32_t)((size_t)ntiles * KB * 4 * a.szw));
  R.z = rsrc(a.zr, (uint32_t)((size_t)ntiles * KB * 4 * a.szw));
  // lane's activation row (token lane % 32) and k half (32 (lane / 32)), in bytes
  const int xoff = ((lane & 31) * a.K + 32 * (lane >> 5)) * 2;

  f32x16 acc[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) acc[p] = f32x16{};

  // Rolling ring of D + 1 block slots: block i sits in slot i mod (D + 1).  Before block i is
  // multiplied, block i + D goes into the slot that block i - 1 freed, so D blocks stay in
  // flight behind the one in use.  Slot indices are compile-time constants (rounds of D + 1
  // blocks are unrolled), which keeps the ring in registers at any K.
  Blk<NP> ring[D + 1];
  auto consume = [&](const Blk<NP>& b, int kb) {
    // exact wave-uniform test: are all zero-points of this block integers (1024 + z exact)?
    bool exact = true;
    const f16x2 c1024 = {(f16)1024.0f, (f16)1024.0f};
#pragma unroll
    for (int p = 0; p < NP; ++p)
      exact = exact && (__builtin_bit_cast(uint32_t, (as_h2(b.zp[p]) + c1024) - c1024) == b.zp[p]);
    const bool half = half_last && kb == KB - 1;
    if (__ballot(exact) == ~0ull)
      block_math<BITS, NP, true>(b, magic, half, acc);
    else
      block_math<BITS, NP, false>(b, magic, half, acc);
  };
  // the first D blocks unconditionally (a wave with fewer blocks re-reads its last one, a wave
  // with none reads block 0 and never uses it)
  const int klast = max(kb1 - 1, 0);
#pragma unroll
  for (int i = 0; i < D; ++i) issue<BITS, NP>(ring[i], R, a, m, pair0, ntiles, min(kb0 + i, klast), xoff);
  // whole rounds whose loads are all in range: unconditional, so the compiler's wait counts
  // stay exact across the loop
  int c = kb0;
  for (; c + 2 * D < kb1; c += D + 1) {
#pragma unroll
    for (int j = 0; j <= D; ++j) {
      issue<BITS, NP>(ring[(j + D) % (D + 1)], R, a, m, pair0, ntiles, c + j + D, xoff);
      consume(ring[j], c + j);
    }
  }
  // the last (at most 2 D) blocks
#pragma unroll
  for (int j = 0; j < 2 * D; ++j) {
    if (c + j + D < kb1) issue<BITS, NP>(ring[(j + D) % (D + 1)], R, a, m, pair0, ntiles, c + j + D, xoff);
    if (c + j < kb1) consume(ring[j % (D + 1)], c + j);
  }

  // fixed-order sum of the NW partials: red[w][p][v][lane]
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[((wave * NP + p) * 16 + v) * 64 + lane] = acc[p][v];
  __syncthreads();
  auto sum = [&](int p, int v) {
    float s = red[((0 * NP + p) * 16 + v) * 64 + lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) s += red[((w * NP + p) * 16 + v) * 64 + lane];
    return s;
  };
  const int h = lane >> 5;
  const int t = lane & 31;
  if (t >= a.T) return;
  if constexpr (EPI == EPI_SWIGLU) {
    for (int idx = wave; idx < NP * 2; idx += NW) {
      const int p = idx >> 1, q = idx & 1;
      const int pair = pair0 + p;
      if (2 * pair >= ntiles) continue;
      const f32x4 g = {sum(p, 4 * q), sum(p, 4 * q + 1), sum(p, 4 * q + 2), sum(p, 4 * q + 3)};
      const f32x4 u = {sum(p, 8 + 4 * q), sum(p, 9 + 4 * q), sum(p, 10 + 4 * q), sum(p, 11 + 4 * q)};
      store_quad<EPI>(a, t, 16 * pair + 8 * q + 4 * h, g, u);
    }
  } else {
    for (int idx = wave; idx < NP * 4; idx += NW) {
      const int p = idx >> 2, q = idx & 3;
      const int pair = pair0 + p;
      if (2 * pair >= ntiles) continue;
      if (q >= 2 && 2 * pair + 1 >= ntiles) continue;  // odd tile count: no second tile
      const f32x4 v = {sum(p, 4 * q), sum(p, 4 * q + 1), sum(p, 4 * q + 2), sum(p, 4 * q + 3)};
      store_quad<EPI>(a, t, 32 * pair + 8 * q + 4 * h, v, f32x4{});
    }
  }
}

constexpr int kNW = 8;  // waves per workgroup (K split)

template <int BITS, int NP, int EPI>
hipError_t run_k(const KArgs& a, hipStream_t stream) {
  const int ntiles = a.rows / 16;
  const int npairs = (ntiles + 1) / 2;
  const int grid = (npairs + NP - 1) / NP;
  const size_t lds = (size_t)kNW * NP * 16 * 64 * 4;
  constexpr int D = NP == 1 ? 3 : 1;  // blocks in flight per wave (register budget)
  return launch_kernel(&splitk_kernel<BITS, NP, kNW, D, EPI>, dim3(grid), dim3(kNW * 64), lds, stream, a);
}

template <int BITS, int EPI>
hipError_t pick_np(const KArgs& a, hipStream_t stream) {
  // two pairs per workgroup (4-bit; the 5-bit ring does not fit twice in registers) while that
  // still leaves a workgroup for most compute units; one pair otherwise
  const int npairs = (a.rows / 16 + 1) / 2;
  if constexpr (BITS == 4) {
    if (npairs >= 2 * 160) return run_k<BITS, 2, EPI>(a, stream);
  }
  return run_k<BITS, 1, EPI>(a, stream);
}

template <int BITS>
hipError_t pick_epi(int epi, const KArgs& a, hipStream_t stream) {
  if (epi == EPI_SWIGLU) return pick_np<BITS, EPI_SWIGLU>(a, stream);
  if (epi == EPI_ADD) return pick_np<BITS, EPI_ADD>(a, stream);
  return pick_np<BITS, EPI_STORE>(a, stream);
}

}  // namespace

hipError_t launch_splitk(int bits, int epi, const KArgs& a, hipStream_t stream) {
  return bits == 5 ? pick_epi<5>(epi, a, stream) : pick_epi<4>(epi, a, stream);
}

}  // namespace w4
