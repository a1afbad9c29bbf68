// Narrow matrix-core path: up to 64 token columns (batched decode, speculative verify).
//
// Prior art: the small-T MMA kernels of the ninfer-3080 performance notes ("What changed":
// permuted k order, activation slabs shared by several row tiles so that they are not re-read
// per tile; "What is left at C8": the T=32 kernel is latency bound, and the lever is operand
// movement and occupancy -- a tile that puts more work in flight).
//
// gfx950 design.  At 17-64 tokens the weight stream still dominates the bytes, the activation
// block (BN tokens x 128 columns, 8-16 KB) is needed by every workgroup, and the matrix-core
// work per weight byte is 4-8x that of decode, so the kernel has to keep a deep stream of code
// loads in flight while the math runs.  One wave's vector-memory counter is in order, so a wave
// that waits for a recent load also waits for every older one; the roles are therefore split
// between waves (warp specialisation), each with only one stream in its counter:
//  * wave 4 streams the packed codes, scales and zero-points of the workgroup's NP 32-row tile
//    pairs, LC blocks ahead, into an LDS ring (buffer_load ... lds: no registers, no copies);
//  * wave 5 streams the activation tile of each block, LX blocks ahead, into a second LDS ring
//    (16-byte chunks XOR-swizzled by token row, conflict-free reads);
//  * waves 0-3 do the math.  The eight 16-k matrix-core steps of every 128-column block are
//    split between them: wave w takes set S = w / 2, dwords 2 (w % 2) and 2 (w % 2) + 1 of each
//    pair's packed block (the packed layout is the operand order of v_mfma_f32_32x32x16_f16 for
//    a 32-row pair), dequantises its 8 bytes per lane per pair in registers and runs NTT
//    matrix-core steps per fragment (B = 32 tokens).
//  * One barrier per block: producers arrive once their loads for the block have landed,
//    consumers once they have finished reading the previous block (its stages are then free).
//    Loads past the last block re-read the last block into free stages, so the per-block load
//    count, and with it every wait, is a compile-time constant.
//  * The four consumers' partial sums are added in a fixed order through LDS (bitwise
//    reproducible), then the epilogue (store / SwiGLU / residual add) writes fp16 quads.
//  * Integer zero-points (checked exactly once per workgroup) select the short dequantisation.
#include "device.h"
#include "kernels.h"
#include "tile32.h"

namespace w4 {
namespace {

using namespace w4dev;
using namespace t32;
using w4layout::block_bytes;

constexpr int kConsumers = 4;
constexpr int kThreads = 64 * (kConsumers + 2);

// Byte layout of one code stage: NP pairs x 2 tiles of 1 KB low-plane codes (64 lanes x 16 B,
// as in the packed block), then (5-bit) 2 NP x 256 B high planes, then 256 B of scale pairs and
// 256 B of zero-point pairs (lane 16 i + r of the load = tile i, row r).
template <int BITS, int NP>
struct CodeStage {
  static constexpr int kLo = 0;
  static constexpr int kHi = NP * 2 * 1024;
  static constexpr int kS = kHi + (BITS == 5 ? NP * 2 * 256 : 0);
  static constexpr int kZ = kS + 256;
  static constexpr int kBytes = kZ + 256;
  // direct-to-LDS instructions the code producer issues per block
  static constexpr int kOps = NP * 2 * (BITS == 5 ? 2 : 1) + 2;
};

// Workgroup barrier without a memory fence.  The fence that __syncthreads() adds would wait for
// every outstanding load of the wave, including the ones meant to stay in flight; the waits are
// explicit instead (producers: vmcnt for their own loads; consumers: lgkmcnt for their LDS
// reads).  The "memory" clobber keeps the compiler from moving memory operations across it.
__device__ __forceinline__ void arrive_wait() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct-to-LDS loads: lane L's bytes land at lds + SIZE * L.
__device__ __forceinline__ void lds_load16(const __amdgpu_buffer_rsrc_t& r, char* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, 0, 0, 0);
}
__device__ __forceinline__ void lds_load4(const __amdgpu_buffer_rsrc_t& r, char* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           voffset, 0, 0, 0);
}

// Codes, high planes, scales and zero-points of block kb for the workgroup's pairs.  Tile
// indices are clamped to the last tile (an odd tile count leaves an empty second tile in the
// last pair; its rows are never stored).
template <int BITS, int NP>
__device__ __forceinline__ void load_codes(const Rsrcs& R, const KArgs& a, char* st, int pair0,
                                           int ntiles, int kb, int lane) {
  using CS = CodeStage<BITS, NP>;
  constexpr int BLK = block_bytes(BITS);
#pragma unroll
  for (int i = 0; i < 2 * NP; ++i) {
    const int tile = min(2 * pair0 + i, ntiles - 1);
    const int bi = tile * a.KB + kb;
    lds_load16(R.w, st + CS::kLo + i * 1024, bi * BLK + lane * 16);
    if constexpr (BITS == 5) lds_load4(R.w, st + CS::kHi + i * 256, bi * BLK + 1024 + lane * 4);
  }
  // scales / zero-points: lane 16 i + r takes tile i, row r (lanes past 2 NP tiles re-read the
  // last tile; their LDS words are never read)
  const int tile = min(2 * pair0 + min(lane >> 4, 2 * NP - 1), ntiles - 1);
  const int off = (tile * a.KB + kb) * 64 + (lane & 15) * 4;
  lds_load4(R.s, st + CS::kS, off);
  lds_load4(R.z, st + CS::kZ, off);
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

// Producer loop: stage (kb + L) % (L + 1) is refilled right after the barrier of block kb, which
// every consumer reaches only after finishing block kb - 1 (the stage's previous contents).
// OPS loads per block; L - 1 blocks of loads may still be in flight when block kb is needed.
template <int L, int OPS, typename Issue>
__device__ __forceinline__ void produce(int KB, Issue issue) {
  constexpr int NWAIT = (L - 1) * OPS;
  static_assert(NWAIT < 64, "vmcnt range");
  for (int kb = 0; kb < KB; ++kb) {
    wait_vmcnt<NWAIT>();  // block kb is in LDS
    arrive_wait();
    issue((kb + L) % (L + 1), min(kb + L, KB - 1));
  }
}

// One consumer: wave W's two k-steps of every block.
template <int BITS, int NP, int NTT, int LC, int LX, int W, bool FAST>
__device__ __forceinline__ void consume(const KArgs& a, const char* cring, const char* xring,
                                        f32x16 (&acc)[NP][NTT]) {
  using CS = CodeStage<BITS, NP>;
  constexpr int BN = 32 * NTT, XB = BN * 256;
  constexpr int J0 = 2 * (W & 1), S = W >> 1;
  const int lane = threadIdx.x & 63;
  const LaneMap m = lane_map(lane);
  const uint32_t magic = vgpr_const(0x64006400u);
  const int brow = lane & 31;
  const int bsw = brow * 256 + 16 * ((4 * (lane >> 5)) ^ (brow & 15));
  const int slot = m.slot16[S];
  // lane-constant byte offsets inside a code stage
  const int lo_off = CS::kLo + m.th * 1024 + slot + 8 * (W & 1);
  const int hi_off = CS::kHi + m.th * 256 + slot / 4;
  const int sz_off = m.th * 64 + m.row4;
  const int KB = a.KB;
  const bool half_last = (KB * 128 != a.K);  // last block holds one group only
  int cst = 0, xst = 0;                       // stage indices of block kb
  for (int kb = 0; kb < KB; ++kb) {
    arrive_wait();  // block kb is in LDS; everyone has finished block kb - 1
    if ((W & 1) == 0 || !(half_last && kb == KB - 1)) {
      const char* cs = cring + cst * CS::kBytes;
      const char* xs = xring + xst * XB;
      u32x2 cw[NP];
      uint32_t hw[NP], sp[NP], zp[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        cw[p] = *reinterpret_cast<const u32x2*>(cs + lo_off + p * 2048);
        hw[p] = BITS == 5 ? *reinterpret_cast<const uint32_t*>(cs + hi_off + p * 512) : 0u;
        sp[p] = *reinterpret_cast<const uint32_t*>(cs + CS::kS + sz_off + p * 128);
        zp[p] = *reinterpret_cast<const uint32_t*>(cs + CS::kZ + sz_off + p * 128);
      }
      f16x8 B0[NTT], B1[NTT];
      load_b<NTT, 2 * J0 + S>(xs, bsw, B0);
      load_b<NTT, 2 * (J0 + 1) + S>(xs, bsw, B1);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const f16x8 A0 = wfrag<BITS, J0, FAST>(cw[p][0], hw[p], magic, zp[p], sp[p]);
        const f16x8 A1 = wfrag<BITS, J0 + 1, FAST>(cw[p][1], hw[p], magic, zp[p], sp[p]);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[p][tt] = mfma32(A0, B0[tt], acc[p][tt]);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[p][tt] = mfma32(A1, B1[tt], acc[p][tt]);
      }
    }
    cst = cst == LC ? 0 : cst + 1;
    xst = xst == LX ? 0 : xst + 1;
  }
}

template <int BITS, int NP, int NTT, int LC, int LX, int W>
__device__ __forceinline__ void consumer(const KArgs& a, const char* cring, const char* xring,
                                         bool fast, f32x16 (&acc)[NP][NTT]) {
  if (fast)
    consume<BITS, NP, NTT, LC, LX, W, true>(a, cring, xring, acc);
  else
    consume<BITS, NP, NTT, LC, LX, W, false>(a, cring, xring, acc);
}

// Workgroup = 4 consumer waves (math) + 1 code producer + 1 activation producer.  LDS: the code
// ring (LC + 1 stages), then the activation ring (LX + 1 stages); the reduction at the end
// reuses the start of it.
template <int BITS, int NP, int NTT, int LC, int LX, int EPI>
__global__ __launch_bounds__(kThreads) void narrow_kernel(KArgs a) {
  using CS = CodeStage<BITS, NP>;
  constexpr int BN = 32 * NTT, XB = BN * 256;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const cring = smem;
  char* const xring = smem + (LC + 1) * CS::kBytes;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = a.rows / 16;
  const int pair0 = blockIdx.x * NP;
  const int KB = a.KB;

  Rsrcs R;
  R.x = rsrc(a.x, (uint32_t)((size_t)a.T * a.K * 2));
  R.w = rsrc(a.w, (uint32_t)((size_t)ntiles * KB * block_bytes(BITS)));
  R.s = rsrc(a.sc, (uint32_t)((size_t)ntiles * KB * 64));
  R.z = rsrc(a.zr, (uint32_t)((size_t)ntiles * KB * 64));
  int voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = lane >> 4;
    voff[i] = (rl * a.K + ((lane & 15) ^ (4 * i + rl)) * 8) * 2;
  }

  // Producers start streaming at once; the consumers vote on the zero-points meanwhile: are all
  // of this workgroup's zero-points integers (1024 + z exact in fp16)?
  bool exact = true;
  if (wave == kConsumers) {
#pragma unroll
    for (int j = 0; j < LC; ++j)
      load_codes<BITS, NP>(R, a, cring + j * CS::kBytes, pair0, ntiles, min(j, KB - 1), lane);
  } else if (wave == kConsumers + 1) {
#pragma unroll
    for (int j = 0; j < LX; ++j) load_x<BN>(R, a, xring + j * XB, voff, min(j, KB - 1));
  } else {
    const int zbase = 2 * pair0 * KB * 64;  // bytes: zero-points of the workgroup's tiles
    const int zbytes = 2 * NP * KB * 64;
    const f16x2 c1024 = {(f16)1024.0f, (f16)1024.0f};
    for (int off = threadIdx.x * 16; off < zbytes; off += 64 * kConsumers * 16) {
      // past the last tile the range check reads zeros (integers)
      const u32x4 zz = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.z, zbase + off, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        exact = exact && (__builtin_bit_cast(uint32_t, (as_h2(zz[e]) + c1024) - c1024) == zz[e]);
    }
  }
  const bool fast = __syncthreads_and(exact);

  f32x16 acc[NP][NTT];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[p][tt] = f32x16{};

  if (wave == kConsumers) {
    produce<LC, CS::kOps>(KB, [&](int st, int kb) {
      load_codes<BITS, NP>(R, a, cring + st * CS::kBytes, pair0, ntiles, kb, lane);
    });
  } else if (wave == kConsumers + 1) {
    produce<LX, BN / 4>(KB, [&](int st, int kb) { load_x<BN>(R, a, xring + st * XB, voff, kb); });
  } else {
    switch (wave) {
      case 0: consumer<BITS, NP, NTT, LC, LX, 0>(a, cring, xring, fast, acc); break;
      case 1: consumer<BITS, NP, NTT, LC, LX, 1>(a, cring, xring, fast, acc); break;
      case 2: consumer<BITS, NP, NTT, LC, LX, 2>(a, cring, xring, fast, acc); break;
      default: consumer<BITS, NP, NTT, LC, LX, 3>(a, cring, xring, fast, acc); break;
    }
  }

  // Drain the producers' tail loads (they target LDS reused below), then add the four partial
  // sums in wave order.  red[w][p][tt][v][lane].
  wait_vmcnt<0>();
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (wave < kConsumers) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[(((wave * NP + p) * NTT + tt) * 16 + v) * 64 + lane] = acc[p][tt][v];
  }
  __syncthreads();
  if (wave >= kConsumers) return;
  auto sum = [&](int p, int tt, int v) {
    float s = red[(((0 * NP + p) * NTT + tt) * 16 + v) * 64 + lane];
    s += red[(((1 * NP + p) * NTT + tt) * 16 + v) * 64 + lane];
    s += red[(((2 * NP + p) * NTT + tt) * 16 + v) * 64 + lane];
    s += red[(((3 * NP + p) * NTT + tt) * 16 + v) * 64 + lane];
    return s;
  };
  const int h = lane >> 5;
  if constexpr (EPI == EPI_SWIGLU) {
    // wave w: gate quad q = w % 2 (its up quad is registers 8 + 4q ..) of the items p*NTT+tt
    // whose parity is w / 2
#pragma unroll
    for (int it = 0; it < NP * NTT; ++it) {
      if ((it & 1) != (wave >> 1)) continue;
      const int p = it / NTT, tt = it % NTT, q = wave & 1;
      const int pair = pair0 + p, t = 32 * tt + (lane & 31);
      if (t >= a.T || 2 * pair >= ntiles) continue;
      const f32x4 g = {sum(p, tt, 4 * q), sum(p, tt, 4 * q + 1), sum(p, tt, 4 * q + 2), sum(p, tt, 4 * q + 3)};
      const f32x4 u = {sum(p, tt, 8 + 4 * q), sum(p, tt, 9 + 4 * q), sum(p, tt, 10 + 4 * q), sum(p, tt, 11 + 4 * q)};
      store_quad<EPI>(a.out, a.res, (size_t)t * a.ldo + 16 * pair + 8 * q + 4 * h, g, u);
    }
  } else {
    // wave w: register quad q = w of every item (pair rows 8q + 4h + 0..3)
    const int q = wave;
#pragma unroll
    for (int it = 0; it < NP * NTT; ++it) {
      const int p = it / NTT, tt = it % NTT;
      const int pair = pair0 + p, t = 32 * tt + (lane & 31);
      if (t >= a.T || 2 * pair >= ntiles) continue;
      if (q >= 2 && 2 * pair + 1 >= ntiles) continue;  // odd tile count: no second tile
      const f32x4 v = {sum(p, tt, 4 * q), sum(p, tt, 4 * q + 1), sum(p, tt, 4 * q + 2), sum(p, tt, 4 * q + 3)};
      store_quad<EPI>(a.out, a.res, (size_t)t * a.ldo + 32 * pair + 8 * q + 4 * h, v, f32x4{});
    }
  }
}

template <int BITS, int NP, int NTT, int EPI>
hipError_t run(const KArgs& a, hipStream_t stream) {
  using CS = CodeStage<BITS, NP>;
  constexpr int BN = 32 * NTT;
  constexpr int LX = 3;  // activation blocks in flight
  constexpr int LCMAX = 63 / CS::kOps + 1;
  constexpr int LC = LCMAX < 12 ? LCMAX : 12;  // code blocks in flight
  const int ntiles = a.rows / 16;
  const int npairs = (ntiles + 1) / 2;
  const int grid = (npairs + NP - 1) / NP;
  const size_t rings = (size_t)(LC + 1) * CS::kBytes + (size_t)(LX + 1) * BN * 256;
  const size_t red = (size_t)kConsumers * NP * NTT * 16 * 64 * 4;
  const size_t lds = rings > red ? rings : red;
  hipLaunchKernelGGL((narrow_kernel<BITS, NP, NTT, LC, LX, EPI>), dim3(grid), dim3(kThreads), lds,
                     stream, a);
  return hipGetLastError();
}

template <int BITS, int NTT, int EPI>
hipError_t pick_np(const KArgs& a, hipStream_t stream) {
  const int ntiles = a.rows / 16;
  const int npairs = (ntiles + 1) / 2;
  // Two pairs per workgroup (each activation block shared by 64 rows) while that still leaves a
  // workgroup for most compute units; one pair otherwise.
  if (npairs >= 2 * 160) return run<BITS, 2, NTT, EPI>(a, stream);
  return run<BITS, 1, NTT, EPI>(a, stream);
}

template <int BITS, int EPI>
hipError_t pick_nt(int tn, const KArgs& a, hipStream_t stream) {
  if (tn <= 32) return pick_np<BITS, 1, EPI>(a, stream);
  return pick_np<BITS, 2, EPI>(a, stream);
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
