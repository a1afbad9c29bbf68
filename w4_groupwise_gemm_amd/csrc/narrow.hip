// Narrow matrix-core path: up to 64 token columns (batched decode, speculative verify).
//
// Prior art: the small-T MMA kernels of the ninfer-3080 performance notes ("What changed":
// permuted k order, activation slabs shared by several row tiles so that they are not re-read
// per tile; "What is left at C8": the T=32 kernel is latency bound, and the lever is operand
// movement and occupancy -- a tile that puts more work in flight).
//
// gfx950 design.  At 17-64 tokens the weight stream still dominates the bytes, the activation
// block (BN tokens x 128 columns, 8-16 KB) is needed by every workgroup, and the matrix-core
// work per weight byte is 4-8x that of decode, so the kernel has to keep a deep stream of loads
// in flight while the math runs.  Every load is a direct-to-LDS buffer load (no registers, no
// copies) into a ring of stages: a block's packed codes, high planes, scales and zero-points
// (the packed layout, copied as is) and its activation tile (16-byte chunks XOR-swizzled by
// token row: conflict-free reads).  One wave's vector-memory counter is in order, so a wave that
// waits for a recent load also waits for every older one; two layouts keep each counter to one
// in-order stream:
//  * producer waves (warp specialisation): wave 4 streams the codes, scales and zero-points of
//    the workgroup's NP 32-row tile pairs DC blocks ahead into a code ring, wave 5 the
//    activation tiles DX blocks ahead into an activation ring; waves 0-3 do the math.  The two
//    rings' depths are independent, which keeps many code bytes in flight when a block's
//    activation tile is large against its codes (one or two pairs, 64 tokens).
//  * self-loading waves (SELF): four waves, one per SIMD (so each may hold up to 512 registers:
//    five pairs of 64-token accumulators fit without spilling), each issuing its share of every
//    block's loads into a common ring of D stages and doing its share of the math.
// In both, the eight 16-k matrix-core steps of every 128-column block are split between the four
// math waves: wave w takes set S = w / 2, dwords 2 (w % 2) and 2 (w % 2) + 1 of each pair's
// packed block (the packed layout is the operand order of v_mfma_f32_32x32x16_f16 for a 32-row
// pair), dequantises its 8 bytes per lane per pair in registers and runs NTT matrix-core steps
// per fragment (B = 32 tokens), reading each block's operands from LDS one block ahead.  One
// fence-free barrier per block: a wave arrives once the loads it waits for have landed and it
// has finished reading the previous block (whose stages are then refilled).  Loads past the last
// block re-read the last block, so the per-block load count, and with it every wait, is a
// compile-time constant.  Rows per workgroup: one or two pairs, or (balanced routes) an even
// share of the row tiles for one workgroup per compute unit, up to five pairs.  The four partial
// sums are added in a fixed order through LDS (bitwise reproducible), then the epilogue (store /
// SwiGLU / residual add) writes fp16 quads.  Integer zero-points (checked exactly once per
// workgroup) select the short dequantisation.
#include "device.h"
#include "kernels.h"
#include "tile32.h"

namespace w4 {
namespace {

using namespace w4dev;
using namespace t32;
using w4layout::block_bytes;

// Byte layout of one code stage: NP pairs x 2 tiles of 1 KB low-plane codes (64 lanes x 16 B,
// as in the packed block), then (5-bit) 2 NP x 256 B high planes, then the scale words and the
// zero-point words of the 2 NP tiles, each tile's (tile, k-block) block in turn (64 bytes, or
// 128 for groups of 32; room is kept for 128).
template <int BITS, int NP>
struct CodeStage {
  static constexpr int kLo = 0;
  static constexpr int kHi = NP * 2 * 1024;
  static constexpr int kS = kHi + (BITS == 5 ? NP * 2 * 256 : 0);
  static constexpr int kZ = kS + NP * 2 * 128;
  static constexpr int kBytes = kZ + NP * 2 * 128;
  // direct-to-LDS instructions the code producer issues per block
  static constexpr int kOps = NP * 2 * (BITS == 5 ? 2 : 1) + 2;
};

// Direct-to-LDS loads: lane L's bytes land at lds + SIZE * L.
__device__ __forceinline__ void lds_load16(const __amdgpu_buffer_rsrc_t& r, char* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, 0, 0, 0);
}
__device__ __forceinline__ void lds_load4(const __amdgpu_buffer_rsrc_t& r, char* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           voffset, 0, 0, 0);
}

// A byte offset past the end of every buffer (all tensors are below 2 GiB): a load from it
// returns zeros without touching memory, and still counts as one load in the wave's counter.
constexpr int kNoLoad = 0x7FFFFFF0;

// Codes, high planes, scales and zero-points of block kb for the workgroup's tiles t0 ..
// t0 + nt - 1 (1 <= nt <= 2 NP).  Stage slots past the workgroup's own tiles (an empty second
// tile in the last pair, or pairs the instance has room for but this workgroup lacks) are
// filled from kNoLoad: the load count per block stays a compile-time constant, no byte is
// fetched for them, and their rows are never stored.
template <int BITS, int NP>
__device__ __forceinline__ void load_codes(const Rsrcs& R, const KArgs& a, char* st, int t0,
                                           int nt, int kb, int lane) {
  using CS = CodeStage<BITS, NP>;
  constexpr int BLK = block_bytes(BITS);
#pragma unroll
  for (int i = 0; i < 2 * NP; ++i) {
    const int bi = (t0 + i) * a.KB + kb;
    lds_load16(R.w, st + CS::kLo + i * 1024, i < nt ? bi * BLK + lane * 16 : kNoLoad);
    if constexpr (BITS == 5)
      lds_load4(R.w, st + CS::kHi + i * 256, i < nt ? bi * BLK + 1024 + lane * 4 : kNoLoad);
  }
  // scales / zero-points: the 2 NP tiles' blocks of szb bytes each, 16 bytes per lane, by the
  // lanes that cover them (at least 8 of the 64: one instruction each, whatever the group size)
  const int szb = 4 * a.szw;
  if (lane * 16 < 2 * NP * szb) {
    const int i = lane * 16 / szb;
    const int off = i < nt ? ((t0 + i) * a.KB + kb) * szb + lane * 16 % szb : kNoLoad;
    lds_load16(R.s, st + CS::kS, off);
    lds_load16(R.z, st + CS::kZ, off);
  }
}

// Activation tile of block kb, BN token rows x 256 bytes: BN / 4 direct-to-LDS instructions of
// 4 rows each.  Lane L of an instruction takes row r0 + L/16 and stores LDS chunk L%16, which
// holds source chunk (L%16) ^ (row & 15).  The whole offset is in the range-checked lane
// operand: token rows beyond T lie past the end of the buffer and read as zero; columns beyond
// K inside the buffer (half-empty last block) read the next row, and those k slots are never
// used by the math.
template <int BN>
__device__ __forceinline__ void load_x(const Rsrcs& R, const KArgs& a, char* xs,
                                       const int (&voff)[4], int kb) {
#pragma unroll
  for (int i = 0; i < BN / 4; ++i) {
    const int r0 = 4 * i;
    lds_load16(R.x, xs + r0 * 256, voff[(r0 & 15) >> 2] + (r0 * a.K + kb * 128) * 2);
  }
}

// Producer loop.  Ring of D stages, block b in stage b % D.  The prologue issued blocks
// 0 .. D-1.  Barrier B(-1) says block 0 is in LDS; barrier B(kb) says block kb + 1 is in LDS
// and that every consumer has finished reading block kb (consumers read one block ahead of
// their math), whose stage is then refilled with block kb + D.  OPS loads per block: D - 2
// blocks of loads may still be in flight at the wait for block kb + 1.
template <int D, int OPS, typename Issue>
__device__ __forceinline__ void produce(int KB, Issue issue) {
  static_assert(D >= 2, "ring too shallow");
  constexpr int NWAIT = (D - 2) * OPS;
  static_assert(NWAIT + OPS < 64, "vmcnt range");
  wait_vmcnt<NWAIT + OPS>();  // block 0
  arrive_wait();              // B(-1)
  for (int kb = 0; kb < KB; ++kb) {
    wait_vmcnt<NWAIT>();  // block kb + 1
    arrive_wait();        // B(kb)
    issue(kb % D, min(kb + D, KB - 1));
  }
}

// Loads of one k-block, split over the NC waves of the workgroup: load j (0 .. kL - 1) is issued
// by wave j % NC into the block's stage (code part cs, activation part xs).  In order: the 2 NP
// low-plane tiles, (5-bit) their 2 NP high planes, the scale words, the zero-point words, then
// the activation tile's BN / 4 loads of 4 token rows each.
template <int BITS, int NP, int BN>
struct BlockLoads {
  static constexpr int kTiles = 2 * NP * (BITS == 5 ? 2 : 1);
  static constexpr int kL = kTiles + 2 + BN / 4;
  static constexpr int per_wave(int w, int nc) { return (kL - w + nc - 1) / nc; }
};

// Wave W's share of block kb's loads.  Stage slots past the workgroup's own tiles read nothing
// (kNoLoad).  Activation tile: lane L of an instruction takes token row r0 + L/16 and stores LDS
// chunk L%16, which holds source chunk (L%16) ^ (row & 15); the whole offset is in the
// range-checked lane operand, so token rows beyond T lie past the end of the buffer and read as
// zero, and columns beyond K inside the buffer (half-empty last block) read the next row,
// whose k slots the math never uses.
template <int BITS, int NP, int BN, int NC, int W>
__device__ __forceinline__ void issue_block(const Rsrcs& R, const KArgs& a, char* cs, char* xs,
                                            const int (&voff)[4], int t0, int nt, int kb, int lane) {
  using CS = CodeStage<BITS, NP>;
  using BL = BlockLoads<BITS, NP, BN>;
  constexpr int BLK = block_bytes(BITS);
#pragma unroll
  for (int j = W; j < BL::kL; j += NC) {
    if (j < 2 * NP) {
      const int bi = (t0 + j) * a.KB + kb;
      lds_load16(R.w, cs + CS::kLo + j * 1024, j < nt ? bi * BLK + lane * 16 : kNoLoad);
    } else if (j < BL::kTiles) {
      const int i = j - 2 * NP;
      const int bi = (t0 + i) * a.KB + kb;
      lds_load4(R.w, cs + CS::kHi + i * 256, i < nt ? bi * BLK + 1024 + lane * 4 : kNoLoad);
    } else if (j < BL::kTiles + 2) {
      // scale (or zero-point) words of the 2 NP tiles, szb bytes each, 16 bytes per lane by the
      // lanes that cover them (at least 8 of the 64, whatever the group size)
      const int szb = 4 * a.szw;
      if (lane * 16 < 2 * NP * szb) {
        const int i = lane * 16 / szb;
        const int off = i < nt ? ((t0 + i) * a.KB + kb) * szb + lane * 16 % szb : kNoLoad;
        if (j == BL::kTiles)
          lds_load16(R.s, cs + CS::kS, off);
        else
          lds_load16(R.z, cs + CS::kZ, off);
      }
    } else {
      const int r0 = 4 * (j - BL::kTiles - 2);
      lds_load16(R.x, xs + r0 * 256, voff[(r0 & 15) >> 2] + (r0 * a.K + kb * 128) * 2);
    }
  }
}

// Steps of wave C among NC: with 4 waves, 2 consecutive 16-k steps (dwords J0, J0+1 of set S of
// every pair's packed block); with 8, one.
template <int NC, int C>
struct Steps {
  static constexpr int kN = 8 / NC;
  static constexpr int kJ0 = NC == 4 ? 2 * (C & 1) : (C & 3);
  static constexpr int kS = NC == 4 ? (C >> 1) : (C >> 2);
};

template <int N>
struct CodeWords;
template <>
struct CodeWords<1> {
  using T = uint32_t;
  static __device__ __forceinline__ uint32_t at(T v, int) { return v; }
};
template <>
struct CodeWords<2> {
  using T = u32x2;
  static __device__ __forceinline__ uint32_t at(T v, int j) { return v[j]; }
};

// Operands of one block for one wave, read from LDS one block ahead of the math.
template <int BITS, int NP, int NTT, int N>
struct Frag {
  typename CodeWords<N>::T cw[NP];
  uint32_t hw[NP], sp[NP], zp[NP];
  f16x8 B[N][NTT];
};

// Byte layout of one ring stage: the code part (CodeStage), then the activation tile.
template <int BITS, int NP, int NTT>
struct Stage {
  static constexpr int kCode = CodeStage<BITS, NP>::kBytes;
  static constexpr int kBytes = kCode + 32 * NTT * 256;
};

// Operand reads and math of math wave C: read() fills a register set from a block's code part
// cs and activation tile xs; math() runs the wave's steps of that block.
template <int BITS, int NP, int NTT, int NC, int C, bool FAST>
struct WaveMath {
  using CS = CodeStage<BITS, NP>;
  using ST = Steps<NC, C>;
  using CWd = CodeWords<ST::kN>;
  using F = Frag<BITS, NP, NTT, ST::kN>;
  uint32_t magic;
  int bsw, lo_off, hi_off, szb, sz_off;

  __device__ __forceinline__ explicit WaveMath(const KArgs& a) {
    const int lane = threadIdx.x & 63;
    const LaneMap m = lane_map(a, lane);
    magic = vgpr_const(0x64006400u);
    const int brow = lane & 31;
    bsw = brow * 256 + 16 * ((4 * (lane >> 5)) ^ (brow & 15));
    const int slot = m.slot16[ST::kS];
    // lane-constant byte offsets inside a code stage
    lo_off = CS::kLo + m.th * 1024 + slot + 4 * ST::kJ0;
    hi_off = CS::kHi + m.th * 256 + slot / 4;
    szb = 4 * a.szw;  // bytes of one tile's scale (or zero-point) block
    sz_off = m.th * szb + m.szoff;
  }
  __device__ __forceinline__ void read(const char* cs, const char* xs, F& f) const {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      f.cw[p] = *reinterpret_cast<const typename CWd::T*>(cs + lo_off + p * 2048);
      f.hw[p] = BITS == 5 ? *reinterpret_cast<const uint32_t*>(cs + hi_off + p * 512) : 0u;
      f.sp[p] = *reinterpret_cast<const uint32_t*>(cs + CS::kS + sz_off + p * 2 * szb);
      f.zp[p] = *reinterpret_cast<const uint32_t*>(cs + CS::kZ + sz_off + p * 2 * szb);
    }
    load_b<NTT, 2 * ST::kJ0 + ST::kS>(xs, bsw, f.B[0]);
    if constexpr (ST::kN == 2) load_b<NTT, 2 * (ST::kJ0 + 1) + ST::kS>(xs, bsw, f.B[ST::kN - 1]);
  }
  __device__ __forceinline__ void math(const F& f, f32x16 (&acc)[NP][NTT]) const {
#pragma unroll
    for (int j = 0; j < ST::kN; ++j) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const f16x8 A = j == 0 ? wfrag<BITS, ST::kJ0, FAST>(CWd::at(f.cw[p], 0), f.hw[p], magic, f.zp[p], f.sp[p])
                               : wfrag<BITS, (ST::kJ0 + 1) & 3, FAST>(CWd::at(f.cw[p], 1), f.hw[p], magic, f.zp[p], f.sp[p]);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[p][tt] = mfma32(A, f.B[j][tt], acc[p][tt]);
      }
    }
  }
  // the second step of waves with J0 = 2 falls in the missing group of a half-empty last block
  static constexpr bool kSkipsHalfBlock = ST::kJ0 >= 2;
};

// Producer layout, math wave C.  Iteration kb: barrier B(kb) (block kb + 1 is in LDS; every
// wave has finished reading block kb), read block kb + 1 into registers, then the math of block
// kb from the registers read one iteration earlier, so the LDS latency hides behind a block of
// matrix-core work.  (Barrier B(-1), block 0 in LDS, was passed by the caller.)
template <int BITS, int NP, int NTT, int NC, int DC, int DX, int C, bool FAST>
__device__ __forceinline__ void consume(const KArgs& a, const char* cring, const char* xring,
                                        f32x16 (&acc)[NP][NTT]) {
  using W = WaveMath<BITS, NP, NTT, NC, C, FAST>;
  constexpr int XB = 32 * NTT * 256;
  const W wm(a);
  const int KB = a.KB;
  const bool half_last = (KB * 128 != a.K);  // last block holds one group only
  // two register sets used in turn (no copies, so the reads of one set never wait for the
  // math of the other)
  typename W::F f0, f1;
  auto step = [&](int kb, typename W::F& mine, typename W::F& other) {
    arrive_wait();  // B(kb)
    if (kb + 1 < KB) wm.read(cring + ((kb + 1) % DC) * W::CS::kBytes, xring + ((kb + 1) % DX) * XB, other);
    if (!W::kSkipsHalfBlock || !(half_last && kb == KB - 1)) wm.math(mine, acc);
  };
  wm.read(cring, xring, f0);
  int kb = 0;
  for (; kb + 1 < KB; kb += 2) {
    step(kb, f0, f1);
    step(kb + 1, f1, f0);
  }
  if (kb < KB) step(kb, f0, f1);
}

// Self-loading layout, wave C.  Ring of D stages, block b in stage b % D.  Iteration kb: wait
// until this wave's loads of block kb + 1 have landed, barrier B(kb) (block kb + 1 complete in
// LDS; every wave has finished reading block kb), refill block kb's stage with block kb + D,
// read block kb + 1 into registers, then the math of block kb.  Blocks 0 .. D-1 were issued
// and barrier B(-1) passed before.
template <int BITS, int NP, int NTT, int NC, int D, int C, bool FAST>
__device__ __forceinline__ void run_wave(const KArgs& a, char* ring, const Rsrcs& R,
                                         const int (&voff)[4], int t0, int nt,
                                         f32x16 (&acc)[NP][NTT]) {
  using W = WaveMath<BITS, NP, NTT, NC, C, FAST>;
  using SG = Stage<BITS, NP, NTT>;
  constexpr int BN = 32 * NTT;
  constexpr int NWAIT = (D - 2) * BlockLoads<BITS, NP, BN>::per_wave(C, NC);
  static_assert(D >= 2, "ring too shallow");
  const W wm(a);
  const int lane = threadIdx.x & 63;
  const int KB = a.KB;
  const bool half_last = (KB * 128 != a.K);
  typename W::F f0, f1;
  auto step = [&](int kb, typename W::F& mine, typename W::F& other) {
    wait_vmcnt<NWAIT>();  // this wave's loads of block kb + 1
    arrive_wait();        // B(kb)
    char* st = ring + (kb % D) * SG::kBytes;
    issue_block<BITS, NP, BN, NC, C>(R, a, st, st + SG::kCode, voff, t0, nt, min(kb + D, KB - 1), lane);
    if (kb + 1 < KB) {
      const char* cs = ring + ((kb + 1) % D) * SG::kBytes;
      wm.read(cs, cs + SG::kCode, other);
    }
    if (!W::kSkipsHalfBlock || !(half_last && kb == KB - 1)) wm.math(mine, acc);
  };
  wm.read(ring, ring + SG::kCode, f0);
  int kb = 0;
  for (; kb + 1 < KB; kb += 2) {
    step(kb, f0, f1);
    step(kb + 1, f1, f0);
  }
  if (kb < KB) step(kb, f0, f1);
}

// Self-loading layout: wave C's share of blocks 0 .. D-1.
template <int BITS, int NP, int NTT, int NC, int D, int C>
__device__ __forceinline__ void prologue(const KArgs& a, char* ring, const Rsrcs& R,
                                         const int (&voff)[4], int t0, int nt) {
  using SG = Stage<BITS, NP, NTT>;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < D; ++j)
    issue_block<BITS, NP, 32 * NTT, NC, C>(R, a, ring + j * SG::kBytes, ring + j * SG::kBytes + SG::kCode,
                                           voff, t0, nt, min(j, a.KB - 1), lane);
}

// Math wave C of either layout: (self-loading) wait for its share of block 0 and pass B(-1)
// (producer layout: passed by the caller), read the zero-point votes, then the main loop with
// the dequantisation they select.
template <int BITS, int NP, int NTT, bool SELF, int D1, int D2, int C>
__device__ __forceinline__ void math_wave(const KArgs& a, char* smem, const Rsrcs& R,
                                          const int (&voff)[4], int t0, int nt, const int* votes,
                                          f32x16 (&acc)[NP][NTT]) {
  constexpr int NC = 4;
  if constexpr (SELF) {
    wait_vmcnt<(D1 - 1) * BlockLoads<BITS, NP, 32 * NTT>::per_wave(C, NC)>();
    arrive_wait();  // B(-1)
  }
  bool fast = true;
#pragma unroll
  for (int c = 0; c < NC; ++c) fast = fast && votes[c] != 0;
  if constexpr (SELF) {
    if (fast)
      run_wave<BITS, NP, NTT, NC, D1, C, true>(a, smem, R, voff, t0, nt, acc);
    else
      run_wave<BITS, NP, NTT, NC, D1, C, false>(a, smem, R, voff, t0, nt, acc);
  } else {
    char* const xring = smem + D1 * CodeStage<BITS, NP>::kBytes;
    if (fast)
      consume<BITS, NP, NTT, NC, D1, D2, C, true>(a, smem, xring, acc);
    else
      consume<BITS, NP, NTT, NC, D1, D2, C, false>(a, smem, xring, acc);
  }
}

// Rows of each workgroup: units of `ut` tiles (1, or 2 for the SwiGLU pair, whose gate and up
// tiles stay together), `units` of them in all.  chunk > 0: workgroup b takes units
// b chunk .. b chunk + chunk - 1; chunk == 0: the units are spread evenly over the grid (sizes
// differ by at most one unit), so a grid of one workgroup per compute unit runs in one round.
struct Part {
  int units, ut, chunk;
};

// Workgroup: 4 math waves, plus (producer layout) a code producer and an activation producer.
// LDS, producer layout: the code ring (D1 = DC stages), the activation ring (D2 = DX stages);
// self-loading layout: the ring of D1 stages.  The zero-point votes sit past the ring(s); the
// reduction at the end reuses all of it.
template <int BITS, int NP, int NTT, bool SELF, int D1, int D2, int EPI>
__global__ __launch_bounds__(SELF ? 256 : 384) void narrow_kernel(KArgs a, Part part) {
  using CS = CodeStage<BITS, NP>;
  using SG = Stage<BITS, NP, NTT>;
  constexpr int NC = 4;
  constexpr int BN = 32 * NTT, XB = BN * 256;
  // token block blockIdx.y: tokens BN y .. BN y + BN - 1 (more than one only when T > BN)
  if (blockIdx.y > 0) {
    const size_t t0 = (size_t)blockIdx.y * BN;
    a.x += t0 * a.K;
    a.out += t0 * a.ldo;
    if (a.res) a.res += t0 * a.ldo;
    if (a.xexp) a.xexp += t0;
    a.T -= (int)t0;
  }
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const cring = smem;
  char* const xring = smem + D1 * CS::kBytes;  // (producer layout)
  int* const votes = reinterpret_cast<int*>(SELF ? smem + D1 * SG::kBytes : xring + D2 * XB);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = a.rows / 16;
  // this workgroup's tiles t0 .. t0 + nt - 1 (1 <= nt <= 2 NP; the host sizes the grid so)
  int u0, u1;
  if (part.chunk > 0) {
    u0 = blockIdx.x * part.chunk;
    u1 = min(u0 + part.chunk, part.units);
  } else {
    u0 = (int)((long long)blockIdx.x * part.units / gridDim.x);
    u1 = (int)((long long)(blockIdx.x + 1) * part.units / gridDim.x);
  }
  const int t0 = u0 * part.ut;
  const int nt = min(u1 * part.ut, ntiles) - t0;
  const int KB = a.KB;

  Rsrcs R;
  R.x = rsrc(a.x, (uint32_t)((size_t)a.T * a.K * 2));
  R.w = rsrc(a.w, (uint32_t)((size_t)ntiles * KB * block_bytes(BITS)));
  R.s = rsrc(a.sc, (uint32_t)((size_t)ntiles * KB * 4 * a.szw));
  R.z = rsrc(a.zr, (uint32_t)((size_t)ntiles * KB * 4 * a.szw));
  int voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = lane >> 4;
    voff[i] = (rl * a.K + ((lane & 15) ^ (4 * i + rl)) * 8) * 2;
  }

  // Producer layout: the producers start streaming at once, the math waves vote on the
  // zero-points meanwhile (are all of this workgroup's zero-points integers, 1024 + z exact in
  // fp16?), and the votes meet in LDS at barrier B(-1), which the producers reach as soon as
  // their first block has landed.  Self-loading layout: each wave's first vote loads go out
  // ahead of its share of the prologue, so that the vote waits only for its own loads (later
  // passes, past 64 KB of zero-points, wait behind the prologue).  Past the last tile the range
  // check reads zeros (integers).
  if (!SELF && wave >= NC) {
    if constexpr (!SELF) {
      if (wave == NC) {
#pragma unroll
        for (int j = 0; j < D1; ++j)
          load_codes<BITS, NP>(R, a, cring + j * CS::kBytes, t0, nt, min(j, KB - 1), lane);
      } else {
#pragma unroll
        for (int j = 0; j < D2; ++j) load_x<BN>(R, a, xring + j * XB, voff, min(j, KB - 1));
      }
    }
  } else {
    const int zbase = t0 * KB * 4 * a.szw;  // bytes: zero-points of the workgroup's tiles
    const int zbytes = nt * KB * 4 * a.szw;
    const f16x2 c1024 = {(f16)1024.0f, (f16)1024.0f};
    constexpr int STEP = 64 * NC * 16;  // bytes per load instruction of the four math waves
    bool exact = true;
    auto pass_load = [&](int off0, u32x4 (&zz)[4]) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        zz[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.z, zbase + off0 + u * STEP, 0, 0));
    };
    auto pass_check = [&](int off0, const u32x4 (&zz)[4]) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          exact = exact && (off0 + u * STEP >= zbytes ||
                            __builtin_bit_cast(uint32_t, (as_h2(zz[u][e]) + c1024) - c1024) == zz[u][e]);
    };
    int off0 = threadIdx.x * 16;
    u32x4 zz[4];
    pass_load(off0, zz);
    if constexpr (SELF) {
      switch (wave) {
        case 0: prologue<BITS, NP, NTT, NC, D1, 0>(a, smem, R, voff, t0, nt); break;
        case 1: prologue<BITS, NP, NTT, NC, D1, 1>(a, smem, R, voff, t0, nt); break;
        case 2: prologue<BITS, NP, NTT, NC, D1, 2>(a, smem, R, voff, t0, nt); break;
        default: prologue<BITS, NP, NTT, NC, D1, 3>(a, smem, R, voff, t0, nt); break;
      }
    }
    pass_check(off0, zz);
    for (off0 += 4 * STEP; off0 < zbytes; off0 += 4 * STEP) {
      pass_load(off0, zz);
      pass_check(off0, zz);
    }
    const bool all = __ballot(exact) == ~0ull;
    if (lane == 0) votes[wave] = all ? 1 : 0;
  }

  f32x16 acc[NP][NTT];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[p][tt] = f32x16{};

  if (!SELF && wave >= NC) {
    if constexpr (!SELF) {
      if (wave == NC)
        produce<D1, CS::kOps>(KB, [&](int st, int kb) {
          load_codes<BITS, NP>(R, a, cring + st * CS::kBytes, t0, nt, kb, lane);
        });
      else
        produce<D2, BN / 4>(KB, [&](int st, int kb) { load_x<BN>(R, a, xring + st * XB, voff, kb); });
    }
  } else {
    if constexpr (!SELF) arrive_wait();  // B(-1): block 0 is in LDS, and so are the votes
    switch (wave) {
      case 0: math_wave<BITS, NP, NTT, SELF, D1, D2, 0>(a, smem, R, voff, t0, nt, votes, acc); break;
      case 1: math_wave<BITS, NP, NTT, SELF, D1, D2, 1>(a, smem, R, voff, t0, nt, votes, acc); break;
      case 2: math_wave<BITS, NP, NTT, SELF, D1, D2, 2>(a, smem, R, voff, t0, nt, votes, acc); break;
      default: math_wave<BITS, NP, NTT, SELF, D1, D2, 3>(a, smem, R, voff, t0, nt, votes, acc); break;
    }
  }

  // Drain the tail loads (they target LDS reused below), then add the four partial sums in wave
  // order.  red[w][p][tt][v][lane].
  wait_vmcnt<0>();
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (wave < NC) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[(((wave * NP + p) * NTT + tt) * 16 + v) * 64 + lane] = acc[p][tt][v];
  }
  __syncthreads();
  if (wave >= NC) return;
  auto sum = [&](int p, int tt, int v) {
    float s = red[(((0 * NP + p) * NTT + tt) * 16 + v) * 64 + lane];
#pragma unroll
    for (int w = 1; w < NC; ++w) s += red[(((w * NP + p) * NTT + tt) * 16 + v) * 64 + lane];
    return s;
  };
  const int h = lane >> 5;
  if constexpr (EPI == EPI_SWIGLU) {
    // (item, gate quad q) pairs, q in {0, 1}; the up quad of gate quad q is registers 8 + 4q ..
    for (int idx = wave; idx < NP * NTT * 2; idx += NC) {
      const int it = idx >> 1, q = idx & 1;
      const int p = it / NTT, tt = it % NTT;
      const int t = 32 * tt + (lane & 31);
      if (t >= a.T || 2 * p >= nt) continue;
      const f32x4 g = {sum(p, tt, 4 * q), sum(p, tt, 4 * q + 1), sum(p, tt, 4 * q + 2), sum(p, tt, 4 * q + 3)};
      const f32x4 u = {sum(p, tt, 8 + 4 * q), sum(p, tt, 9 + 4 * q), sum(p, tt, 10 + 4 * q), sum(p, tt, 11 + 4 * q)};
      store_quad<EPI>(a, t, 8 * (t0 + 2 * p) + 8 * q + 4 * h, g, u);
    }
  } else {
    // (item, register quad q) pairs: pair rows 8q + 4h + 0..3
    for (int idx = wave; idx < NP * NTT * 4; idx += NC) {
      const int it = idx >> 2, q = idx & 3;
      const int p = it / NTT, tt = it % NTT;
      const int t = 32 * tt + (lane & 31);
      if (t >= a.T || 2 * p + (q >> 1) >= nt) continue;  // no such tile in this workgroup
      const f32x4 v = {sum(p, tt, 4 * q), sum(p, tt, 4 * q + 1), sum(p, tt, 4 * q + 2), sum(p, tt, 4 * q + 3)};
      store_quad<EPI>(a, t, 16 * (t0 + 2 * p) + 8 * q + 4 * h, v, f32x4{});
    }
  }
}

// Producer layout: code ring as deep as the code producer's load counter allows (at most 12),
// activation ring likewise for the activation producer.  Self-loading layout: as many stages as
// the LDS holds, within each wave's load counter, at most 16.
template <int BITS, int NP, int NTT, bool SELF, int EPI>
hipError_t run(const KArgs& a, int grid, Part part, hipStream_t stream) {
  using CS = CodeStage<BITS, NP>;
  using SG = Stage<BITS, NP, NTT>;
  constexpr int NC = 4;
  constexpr int BN = 32 * NTT;
  constexpr int kLds = 160 * 1024;
  constexpr int DCMAX = 63 / CS::kOps + 1;
  constexpr int DX = 63 / (BN / 4) + 1;
  constexpr int NMAX = BlockLoads<BITS, NP, BN>::per_wave(0, NC);
  constexpr int D_LDS = (kLds - NC * (int)sizeof(int)) / SG::kBytes;
  constexpr int D_CNT = 63 / NMAX + 1;
  constexpr int D_SELF = D_LDS < D_CNT ? (D_LDS < 16 ? D_LDS : 16) : (D_CNT < 16 ? D_CNT : 16);
  constexpr int D1 = SELF ? D_SELF : (DCMAX < 12 ? DCMAX : 12);
  constexpr int D2 = SELF ? 0 : DX;
  constexpr size_t rings = SELF ? (size_t)D1 * SG::kBytes + NC * sizeof(int)
                                : (size_t)D1 * CS::kBytes + (size_t)D2 * BN * 256 + NC * sizeof(int);
  constexpr size_t red = (size_t)NC * NP * NTT * 16 * 64 * 4;
  constexpr size_t lds = rings > red ? rings : red;
  static_assert(lds <= kLds, "LDS of one workgroup");
  const int ntb = (a.T + BN - 1) / BN;
  if (ntb > 65535) return hipErrorInvalidConfiguration;  // grid y limit (T above 4 million)
  return launch_kernel(&narrow_kernel<BITS, NP, NTT, SELF, D1, D2, EPI>, dim3(grid, ntb),
                       dim3(SELF ? 256 : 384), lds, stream, a, part);
}

constexpr int kCUs = 256;    // compute units of the chip (gfx950, MI350 series)
constexpr int kMaxPairs = 5;  // largest instance (pairs per workgroup)

template <int BITS, int NTT, int EPI>
hipError_t pick_np(bool balanced, const KArgs& a, hipStream_t stream) {
  const int ntiles = a.rows / 16;
  if (!balanced) {
    // Two pairs per workgroup (each activation block shared by 64 rows) while that still
    // leaves a workgroup for most compute units; one pair otherwise.
    const int npairs = (ntiles + 1) / 2;
    const int np = npairs >= 2 * 160 ? 2 : 1;
    const int grid = (npairs + np - 1) / np;
    const Part part{npairs, 2, np};
    return np == 2 ? run<BITS, 2, NTT, false, EPI>(a, grid, part, stream)
                   : run<BITS, 1, NTT, false, EPI>(a, grid, part, stream);
  }
  // Balanced: one workgroup per compute unit (fewer when there are fewer units), each with an
  // even share of the units; more workgroups only when a share would exceed kMaxPairs pairs.
  const int ut = EPI == EPI_SWIGLU ? 2 : 1;
  const int units = ntiles / ut;
  const int cap = 2 * kMaxPairs / ut;  // units per workgroup
  int grid = units < kCUs ? units : kCUs;
  if ((units + grid - 1) / grid > cap) grid = (units + cap - 1) / cap;
  const int per = (units + grid - 1) / grid;  // largest share
  const int np = (per * ut + 1) / 2;
  const Part part{units, ut, 0};
  // Layout: self-loading for 64-token tiles over three or more pairs (the SwiGLU pair at
  // 17408 x 2 rows, T = 64: 45.1 against 51.7 us with producer waves, whose five-pair 64-token
  // instance spills); producer waves otherwise, where a block's activation tile is large against
  // its codes (one or two pairs) or the 32-token instances fit anyway (T = 32: 31.7 against
  // 34.2 us self-loading).
  constexpr bool kSelf = NTT == 2;
  switch (np) {
    case 1: return run<BITS, 1, NTT, false, EPI>(a, grid, part, stream);
    case 2: return run<BITS, 2, NTT, false, EPI>(a, grid, part, stream);
    case 3: return run<BITS, 3, NTT, kSelf, EPI>(a, grid, part, stream);
    case 4: return run<BITS, 4, NTT, kSelf, EPI>(a, grid, part, stream);
    default: return run<BITS, 5, NTT, kSelf, EPI>(a, grid, part, stream);
  }
}

template <int BITS, int EPI>
hipError_t pick_nt(int tn, bool balanced, const KArgs& a, hipStream_t stream) {
  if (tn <= 32) return pick_np<BITS, 1, EPI>(balanced, a, stream);
  return pick_np<BITS, 2, EPI>(balanced, a, stream);
}

template <int BITS>
hipError_t pick_epi(int tn, bool balanced, int epi, const KArgs& a, hipStream_t stream) {
  if (epi == EPI_SWIGLU) return pick_nt<BITS, EPI_SWIGLU>(tn, balanced, a, stream);
  if (epi == EPI_ADD) return pick_nt<BITS, EPI_ADD>(tn, balanced, a, stream);
  return pick_nt<BITS, EPI_STORE>(tn, balanced, a, stream);
}

}  // namespace

// One object per code width (W4_NARROW_BITS), so that the two compile in parallel.
#if W4_NARROW_BITS == 4
hipError_t launch_narrow_b4(int tn, bool balanced, int epi, const KArgs& a, hipStream_t stream) {
  return pick_epi<4>(tn, balanced, epi, a, stream);
}
#elif W4_NARROW_BITS == 5
hipError_t launch_narrow_b5(int tn, bool balanced, int epi, const KArgs& a, hipStream_t stream) {
  return pick_epi<5>(tn, balanced, epi, a, stream);
}
#else
#error "compile narrow.hip with -DW4_NARROW_BITS=4 or 5"
#endif

}  // namespace w4
