// A8 prefill route: int8 activations with a scale per 64 columns, int8 matrix-core steps, and
// the per-group rescale of the int32 partial sums into fp32.  Lossy, by definition of the route.
//
// The route of the ninfer-3080 performance notes ("A8 prefill routes"; accuracy held to a
// relative L2 error of 0.04 against an fp64 oracle, 0.010-0.020 measured; the per-group rescale
// and the scale reads are about a sixth of their kernel: "The token tile, and why it was
// hiding").  The quantisation reading: per token row and 64-column group, s = max |x| / 127 and
// q = rint(x / s) clamped to [-127, 127], in fp32; a group of zeros has s = 0.
//
// gfx950 design.
//  * a8_quant_kernel: one wave per 512 columns of one token row, 8 values per lane, the group
//    maximum from three lane exchanges.  Codes are written in the order the weight unpacking
//    below produces (each 8-column chunk as columns 0 4 1 5 2 6 3 7), so that a lane's 16
//    activation bytes and the 16 weight bytes it multiplies them with are one contiguous load
//    each; the scales are written k-block major ([ceil(K/128)][T][2]), so that one workgroup's
//    128 tokens of one k-block are 1 KB in one place.
//  * a8_kernel: workgroup = 4 waves x one 32-row tile pair each (128 rows) x 128 tokens.  The
//    matrix-core step is v_mfma_i32_32x32x32_i8 with the activations as the A operand and the
//    weights as B, so that a lane's output column is its own weight row and its weight scale
//    is its own fp16 pair.  A step covers the lane-group half of 16 columns x 2 halves that the
//    packed layout gives each lane (two code dwords), so every step stays inside one 64-column
//    group: two steps (code sets 0 and 1) make a group's int32 partial sum P, which is rescaled
//    into the fp32 accumulator as acc += (s_w * s_x) * float(P).
//  * weights to int8: (q | 0x80) - z per byte (no borrow: 128 + q >= 128 > z), then the sign
//    bit flipped: q - z as signed int8, from the nibbles with one and_or per four codes (plus
//    the high plane's bit 4 for 5-bit codes).  Integer zero-points in [0, 127] are required; a
//    workgroup that meets another zero-point writes NaN to its outputs (checked once, exactly).
//  * activation tiles (16 KB of int8 codes and 1 KB of scales per k-block) go straight from
//    memory to LDS, double buffered, 16-byte chunks XOR-swizzled by token row; the weight codes
//    go from memory to registers, one block ahead.
#include <math.h>

#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "tile32.h"

namespace w4 {
namespace {

using namespace w4dev;
using namespace t32;
using w4layout::block_bytes;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kNTT = 4;           // 32-token tiles per workgroup
constexpr int kBN = 32 * kNTT;    // tokens per workgroup
constexpr int kXT = kBN * 128;    // bytes of one int8 activation tile (128 columns)
constexpr int kST = kBN * 2 * 4;  // bytes of its scales (two groups per token)
constexpr int kStage = kXT + kST;

// ---- quantisation

__global__ __launch_bounds__(64) void a8_quant_kernel(const _Float16* __restrict__ x, int T, int K,
                                                      int8_t* __restrict__ xq, float* __restrict__ sx) {
  const int lane = threadIdx.x;
  const int t = blockIdx.y;
  const int c = blockIdx.x * 512 + lane * 8;  // first of this lane's 8 columns
  const bool on = c < K;                       // K % 64 == 0: a group is wholly on or off
  f16x8 v = {};
  if (on) v = *reinterpret_cast<const f16x8*>(x + (size_t)t * K + c);
  float f[8];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[i] = (float)v[i];
    m = fmaxf(m, fabsf(f[i]));
  }
  // the group's 8 lanes are adjacent: lanes 8 j .. 8 j + 7
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float s = m / 127.0f;
  int q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float r = s > 0.f ? rintf(f[i] / s) : 0.f;
    r = fminf(fmaxf(r, -127.f), 127.f);
    q[i] = (int)r;
  }
  if (!on) return;
  // bytes in the order 0 4 1 5 | 2 6 3 7 (the weight unpacking's order)
  auto b = [&](int i) { return (uint32_t)(q[i] & 0xFF); };
  const uint32_t w0 = b(0) | (b(4) << 8) | (b(1) << 16) | (b(5) << 24);
  const uint32_t w1 = b(2) | (b(6) << 8) | (b(3) << 16) | (b(7) << 24);
  *reinterpret_cast<u32x2*>(xq + (size_t)t * K + c) = u32x2{w0, w1};
  if ((lane & 7) == 0) {
    const int g = c / 64;
    sx[((size_t)(g >> 1) * T + t) * 2 + (g & 1)] = s;
    // K % 128 == 64: the last k-block's second group is padding; its scale is written as 0
    if ((g & 1) == 0 && c + 64 == K) sx[((size_t)(g >> 1) * T + t) * 2 + 1] = 0.f;
  }
}

// ---- the matrix kernel

struct A8Codes {
  u32x4 cw[2];   // code slots of sets 0 and 1
  uint32_t hw[2];
  uint32_t sp, zp;  // fp16 scale / zero-point pairs of this lane's row (the block's two groups)
};

template <int BITS>
__device__ __forceinline__ void a8_load_codes(A8Codes& c, const Rsrcs& R, const KArgs& a,
                                              const LaneMap& m, int pair, int ntiles, int kb) {
  constexpr int BLK = block_bytes(BITS);
  const int tile = min(2 * pair + m.th, ntiles - 1);
  const int bi = tile * a.KB + kb;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    c.cw[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.w, bi * BLK + m.slot16[s], 0, 0));
    c.hw[s] = BITS == 5 ? __builtin_amdgcn_raw_buffer_load_b32(R.w, bi * BLK + 1024 + m.slot16[s] / 4, 0, 0) : 0u;
  }
  c.sp = __builtin_amdgcn_raw_buffer_load_b32(R.s, bi * 4 * a.szw + m.szoff, 0, 0);
  c.zp = __builtin_amdgcn_raw_buffer_load_b32(R.z, bi * 4 * a.szw + m.szoff, 0, 0);
}

// Activation tile of k-block kb into LDS: 128 token rows x 128 bytes (16 instructions of 8 rows;
// lane L takes row r0 + L / 8 and stores chunk L % 8, which holds source chunk (L % 8) ^ (row % 8)),
// then the 1 KB of scales (lane L: tokens tok0 + 2 L, + 1, both groups).  Rows past T and
// columns past the end read as zero.
__device__ __forceinline__ void a8_load_x(const Rsrcs& R, __amdgpu_buffer_rsrc_t rsx, const KArgs& a,
                                          char* st, int tok0, int kb, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r0 = (4 * wave + i) * 8;
    const int row = r0 + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        R.x, (__attribute__((address_space(3))) void*)(st + r0 * 128), 16,
        (tok0 + row) * a.K + kb * 128 + chunk * 16, 0, 0, 0);
  }
  if (wave == 0)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, (__attribute__((address_space(3))) void*)(st + kXT), 16,
                                             ((kb * a.T) + tok0 + 2 * lane) * 8, 0, 0, 0);
}

// int8 (q - z) of code dwords j0, j0 + 1 of one set: 16 bytes, columns in the order
// [0 4 1 5 2 6 3 7] of each 8-column run.  zb: the group's zero-point in every byte.
template <int BITS, int J0>
__device__ __forceinline__ i32x4 a8_weights(u32x4 cw, uint32_t hiw, uint32_t zb) {
  i32x4 out;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t w = cw[J0 + d];
    uint32_t lo = and_or(w, 0x0F0F0F0Fu, 0x80808080u);
    uint32_t hi = and_or(w >> 4, 0x0F0F0F0Fu, 0x80808080u);
    if constexpr (BITS == 5) {
      constexpr int tj0 = J0 == 0 ? 0 : 8;  // high-plane offsets of dwords 0 1 2 3: 0 2 8 10
      const uint32_t h = hiw >> (tj0 + 2 * d);  // bit 4 of slots 0 4 1 5 at bits 0 1 16 17, of 2 6 3 7 at 4 5 20 21
      lo = lo | ((h << 4) & 0x00100010u) | ((h << 11) & 0x10001000u);
      hi = hi | (h & 0x00100010u) | ((h << 7) & 0x10001000u);
    }
    out[2 * d] = (int)((lo - zb) ^ 0x80808080u);
    out[2 * d + 1] = (int)((hi - zb) ^ 0x80808080u);
  }
  return out;
}

__device__ __forceinline__ uint32_t byte4(uint32_t v) { return v * 0x01010101u; }

template <int BITS, int EPI>
__global__ __launch_bounds__(256, 2) void a8_kernel(KArgs a, const float* sx, int nrb, int ntb) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = a.rows / 16;
  // XCD-aware order (as the fp16 wide kernel): XCD x takes a contiguous run of tiles
  const int G = nrb * ntb;
  const int b = blockIdx.x, xcd = b % kXCD, l = b / kXCD;
  const int q = G / kXCD, rem = G % kXCD;
  const int t_idx = xcd * q + min(xcd, rem) + l;
  const int rb = t_idx % nrb, tb = t_idx / nrb;
  const int tok0 = tb * kBN;
  const int pair = rb * 4 + wave;
  const LaneMap m = lane_map(a, lane);
  const int h = lane >> 5;

  Rsrcs R;
  R.x = rsrc(a.x, (uint32_t)((size_t)a.T * a.K));  // int8 codes [T][K]
  R.w = rsrc(a.w, (uint32_t)((size_t)ntiles * a.KB * block_bytes(BITS)));
  R.s = rsrc(a.sc, (uint32_t)((size_t)ntiles * a.KB * 4 * a.szw));
  R.z = rsrc(a.zr, (uint32_t)((size_t)ntiles * a.KB * 4 * a.szw));
  const __amdgpu_buffer_rsrc_t rsx = rsrc(sx, (uint32_t)((size_t)a.KB * a.T * 8));

  // Are all zero-points of this workgroup's rows integers in [0, 127]?
  bool ok = true;
  {
    const int zbase = rb * 8 * a.KB * 4 * a.szw, zbytes = 8 * a.KB * 4 * a.szw;
    for (int off = threadIdx.x * 16; off < zbytes; off += 256 * 16) {
      const u32x4 zz = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.z, zbase + off, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2 z2 = as_h2(zz[e]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float zf = (float)z2[i];
          ok = ok && zf >= 0.f && zf <= 127.f && zf == rintf(zf);
        }
      }
    }
  }
  ok = __syncthreads_and(ok);

  i32x16 zero = {};
  float acc[kNTT][16];  // (scalars, not vectors: element-wise updates of vector values kept copies)
#pragma unroll
  for (int tt = 0; tt < kNTT; ++tt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[tt][v] = 0.f;

  a8_load_x(R, rsx, a, smem, tok0, 0, wave, lane);
  A8Codes cur, nxt;
  a8_load_codes<BITS>(cur, R, a, m, pair, ntiles, 0);
  const int brow = lane & 31;
  for (int kb = 0; kb < a.KB; ++kb) {
    wait_vmcnt<0>();
    __syncthreads();
    // the next block's loads, issued unconditionally (the last iteration re-reads the last block
    // into the free buffer) so that the loop body is one basic block the scheduler can order
    const int kn = min(kb + 1, a.KB - 1);
    a8_load_x(R, rsx, a, smem + ((kb + 1) & 1) * kStage, tok0, kn, wave, lane);
    a8_load_codes<BITS>(nxt, R, a, m, pair, ntiles, kn);
    const char* st = smem + (kb & 1) * kStage;
    const float* sxl = reinterpret_cast<const float*>(st + kXT);  // [token][2]
    // (a half-empty last block's second group is the packed padding: codes 0, zero-point 0 and
    // scale 0, so its partial sums are 0 and its activation scale, written as 0, adds nothing)
    // weights of both groups (code sets 0 and 1 each) as int8, and their scales
    const uint32_t zb0 = byte4((uint32_t)(int)(float)as_h2(cur.zp)[0]);
    const uint32_t zb1 = byte4((uint32_t)(int)(float)as_h2(cur.zp)[1]);
    const i32x4 W00 = a8_weights<BITS, 0>(cur.cw[0], cur.hw[0], zb0);
    const i32x4 W01 = a8_weights<BITS, 0>(cur.cw[1], cur.hw[1], zb0);
    const i32x4 W10 = a8_weights<BITS, 2>(cur.cw[0], cur.hw[0], zb1);
    const i32x4 W11 = a8_weights<BITS, 2>(cur.cw[1], cur.hw[1], zb1);
    const float sw0 = (float)as_h2(cur.sp)[0], sw1 = (float)as_h2(cur.sp)[1];
    // token tile by token tile: the two steps of each group (code sets 0 and 1) give its int32
    // partial sums, which are rescaled with the tile's activation scales (read once for both
    // groups); the lane holds tokens 32 tt + 8 (v / 4) + 4 h + v % 4 of its weight row
#pragma unroll
    for (int tt = 0; tt < kNTT; ++tt) {
      const int row = 32 * tt + brow;
      const char* xr = st + row * 128;
      // chunk 4 g + S + 2 h of the token row, stored at chunk ^ (row % 8)
      auto xf = [&](int c) { return *reinterpret_cast<const i32x4*>(xr + ((c ^ (row & 7)) << 4)); };
      i32x16 P0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf(0 + 2 * h), W00, zero, 0, 0, 0);
      P0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf(1 + 2 * h), W01, P0, 0, 0, 0);
      i32x16 P1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf(4 + 2 * h), W10, zero, 0, 0, 0);
      P1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf(5 + 2 * h), W11, P1, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t0 = 32 * tt + 8 * i + 4 * h;
        const f32x4 s01 = *reinterpret_cast<const f32x4*>(sxl + 2 * t0);      // tokens t0, t0 + 1
        const f32x4 s23 = *reinterpret_cast<const f32x4*>(sxl + 2 * t0 + 4);  // t0 + 2, t0 + 3
        const float sxa[4] = {s01[0], s01[2], s23[0], s23[2]};  // group 0 of tokens t0 .. t0 + 3
        const float sxb[4] = {s01[1], s01[3], s23[1], s23[3]};  // group 1
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float y = fmaf(sw0 * sxa[j], (float)P0[4 * i + j], acc[tt][4 * i + j]);
          y = fmaf(sw1 * sxb[j], (float)P1[4 * i + j], y);
          acc[tt][4 * i + j] = y;
        }
      }
      // one tile's partial sums at a time (hoisting every tile's steps ahead of the rescales
      // holds four tiles' partial sums and spills)
      __builtin_amdgcn_sched_barrier(0);
    }
    cur = nxt;
  }

  // epilogue: lane (weight row 32 pair + lane % 32) holds tokens 32 tt + 8 (v / 4) + 4 h + v % 4
  const int rowin = lane & 31;
  const bool tile_ok = 2 * pair + (rowin >> 4) < ntiles;
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int tt = 0; tt < kNTT; ++tt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int t = tok0 + 32 * tt + 8 * (v >> 2) + 4 * h + (v & 3);
      float y = ok ? acc[tt][v] : nan;
      if constexpr (EPI == EPI_SWIGLU) {
        // gate row r in lane r, up row r in lane r + 16 (same half)
        const float up = __shfl_down(y, 16, 32);
        if (rowin < 16 && t < a.T && 2 * pair < ntiles) store_one<EPI>(a, t, 16 * pair + rowin, y, up);
      } else {
        if (t < a.T && tile_ok) store_one<EPI>(a, t, 32 * pair + rowin, y, 0.f);
      }
    }
  }
}

template <int BITS, int EPI>
hipError_t run_a8(const KArgs& a, const float* sx, hipStream_t stream) {
  const int ntiles = a.rows / 16;
  const int nrb = (ntiles + 7) / 8;
  const int ntb = (a.T + kBN - 1) / kBN;
  return launch_kernel(&a8_kernel<BITS, EPI>, dim3(nrb * ntb), dim3(256), (size_t)2 * kStage, stream, a,
                       sx, nrb, ntb);
}

}  // namespace

hipError_t launch_a8_quant(const _Float16* x, int T, int K, int8_t* xq, float* sx, hipStream_t stream) {
  if (T < 1 || K % 64) return hipErrorInvalidValue;
  return launch_kernel(&a8_quant_kernel, dim3((K + 511) / 512, T), dim3(64), 0, stream, x, T, K, xq, sx);
}

hipError_t launch_a8(int bits, int epi, const KArgs& a, const float* sx, hipStream_t stream) {
  if (bits == 5) {
    if (epi == EPI_SWIGLU) return run_a8<5, EPI_SWIGLU>(a, sx, stream);
    if (epi == EPI_ADD) return run_a8<5, EPI_ADD>(a, sx, stream);
    return run_a8<5, EPI_STORE>(a, sx, stream);
  }
  if (epi == EPI_SWIGLU) return run_a8<4, EPI_SWIGLU>(a, sx, stream);
  if (epi == EPI_ADD) return run_a8<4, EPI_ADD>(a, sx, stream);
  return run_a8<4, EPI_STORE>(a, sx, stream);
}

}  // namespace w4
