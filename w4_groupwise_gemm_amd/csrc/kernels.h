// Internal interface between the C ABI (api.hip) and the kernel families.  Plain pointers and
// sizes only; every pointer has been validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

template <typename T>
struct same_type {
  using type = T;
};

// Enqueue one kernel on `stream` and return the status of this launch itself (hipLaunchKernel's
// return value), so that an error left behind by unrelated earlier work is not reported as
// this call's failure.  The arguments are converted to the kernel's parameter types.
template <typename... P>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds,
                                hipStream_t stream, typename same_type<P>::type... args) {
  void* argv[sizeof...(P) + 1] = {static_cast<void*>(&args)..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds, stream);
}

struct KArgs {
  const _Float16* x;     // [T][K] activations (fp16; bf16 inputs arrive here converted)
  const uint8_t* w;      // packed codes, `rows` packed rows
  const uint32_t* sc;    // packed scales: szw fp16 pairs per (row tile, k-block)
  const uint32_t* zr;    // packed zero-points, same layout
  const _Float16* res;   // [T][ldo] residual (EPI_ADD) or nullptr; bf16 bits when xexp is set
  _Float16* out;         // [T][ldo]; bf16 bits when xexp is set
  int T;                 // tokens (>= 1)
  int rows;              // packed rows (2N for the SwiGLU pair)
  int K;                 // columns of X and W
  int KB;                // ceil(K / 128)
  int ldo;               // output columns (N)
  int szw;               // 32-bit scale / zero-point words per (row tile, k-block): 16, or 32 for groups of 32
  const int* xexp;       // bf16 activations: x holds X[t] * 2^-xexp[t] in fp16, and out / res are
                         // bf16 (the epilogue scales by 2^xexp[t]); nullptr for fp16 in and out
};

// Word, inside the scale / zero-point block of a (row tile, k-block), of the pair that row r
// needs when its codes come from lane group g (see w4layout::sz_word).
__device__ __forceinline__ int sz_lane_word(const KArgs& a, int r, int g) {
  return a.szw == 32 ? 16 * (g >> 1) + r : r;
}

// Several matrices sharing one activation (same x, T and K), each with its own output.
constexpr int kMaxParents = 4;
struct GroupedArgs {
  KArgs a[kMaxParents];   // per matrix: x, w, sc, zr, out, T, rows, K, KB, ldo (res unused)
  int bits[kMaxParents];  // 4 or 5
  int n;                  // 1 .. kMaxParents
};

// Each launcher enqueues exactly one kernel on `stream` and returns hipSuccess or the launch
// error.  `epi` is one of w4dev::EPI_*.
// streaming kernel over all matrices of a group in one launch (store epilogue; T <= 64,
// K <= 5120); defined in the 4-bit store part of stream.hip
hipError_t launch_grouped(const GroupedArgs& g, hipStream_t stream);

// streaming kernel (stream.hip, one object per code width b and epilogue e)
#define W4_STREAM_PART(b, e)                                                    \
  hipError_t launch_gemv_b##b##_e##e(const KArgs& a, hipStream_t stream);     \
  hipError_t launch_stream16_b##b##_e##e(const KArgs& a, hipStream_t stream); \
  hipError_t launch_stream32_b##b##_e##e(const KArgs& a, hipStream_t stream); \
  hipError_t launch_stream64_b##b##_e##e(const KArgs& a, hipStream_t stream);
W4_STREAM_PART(4, 0) W4_STREAM_PART(4, 1) W4_STREAM_PART(4, 2)
W4_STREAM_PART(5, 0) W4_STREAM_PART(5, 1) W4_STREAM_PART(5, 2)
#undef W4_STREAM_PART

inline hipError_t launch_gemv(int bits, int epi, const KArgs& a, hipStream_t stream) {  // 1 <= T <= 4
  switch (bits * 4 + epi) {
    case 16: return launch_gemv_b4_e0(a, stream);
    case 17: return launch_gemv_b4_e1(a, stream);
    case 18: return launch_gemv_b4_e2(a, stream);
    case 20: return launch_gemv_b5_e0(a, stream);
    case 21: return launch_gemv_b5_e1(a, stream);
    case 22: return launch_gemv_b5_e2(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// T <= 32, K <= 5120 (two-block ring of 32-row activation tiles)
inline hipError_t launch_stream32(int bits, int epi, const KArgs& a, hipStream_t stream) {
  switch (bits * 4 + epi) {
    case 16: return launch_stream32_b4_e0(a, stream);
    case 17: return launch_stream32_b4_e1(a, stream);
    case 18: return launch_stream32_b4_e2(a, stream);
    case 20: return launch_stream32_b5_e0(a, stream);
    case 21: return launch_stream32_b5_e1(a, stream);
    case 22: return launch_stream32_b5_e2(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// T <= 64, K <= 5120 (one-slot ring of 64-row activation tiles)
inline hipError_t launch_stream64(int bits, int epi, const KArgs& a, hipStream_t stream) {
  switch (bits * 4 + epi) {
    case 16: return launch_stream64_b4_e0(a, stream);
    case 17: return launch_stream64_b4_e1(a, stream);
    case 18: return launch_stream64_b4_e2(a, stream);
    case 20: return launch_stream64_b5_e0(a, stream);
    case 21: return launch_stream64_b5_e1(a, stream);
    case 22: return launch_stream64_b5_e2(a, stream);
    default: return hipErrorInvalidValue;
  }
}

inline hipError_t launch_stream16(int bits, int epi, const KArgs& a, hipStream_t stream) {  // T <= 16
  switch (bits * 4 + epi) {
    case 16: return launch_stream16_b4_e0(a, stream);
    case 17: return launch_stream16_b4_e1(a, stream);
    case 18: return launch_stream16_b4_e2(a, stream);
    case 20: return launch_stream16_b5_e0(a, stream);
    case 21: return launch_stream16_b5_e1(a, stream);
    case 22: return launch_stream16_b5_e2(a, stream);
    default: return hipErrorInvalidValue;
  }
}
// narrow: token tiles of tn (32 or 64) columns; T > tn runs ceil(T / tn) token blocks side by
// side.  balanced: rows spread evenly over one workgroup per compute unit (up to 5 tile pairs
// each); otherwise one or two pairs per workgroup.
hipError_t launch_narrow_b4(int tn, bool balanced, int epi, const KArgs& a, hipStream_t stream);
hipError_t launch_narrow_b5(int tn, bool balanced, int epi, const KArgs& a, hipStream_t stream);
inline hipError_t launch_narrow(int tn, bool balanced, int bits, int epi, const KArgs& a,
                                hipStream_t stream) {
  return bits == 5 ? launch_narrow_b5(tn, balanced, epi, a, stream)
                   : launch_narrow_b4(tn, balanced, epi, a, stream);
}
// register-ring kernel (regring.hip): T <= tn (16, 32 or 64) tokens, any K; row tiles spread
// evenly over one workgroup per compute unit
hipError_t launch_regring_b4(int tn, int epi, const KArgs& a, hipStream_t stream);
hipError_t launch_regring_b5(int tn, int epi, const KArgs& a, hipStream_t stream);
inline hipError_t launch_regring(int tn, int bits, int epi, const KArgs& a, hipStream_t stream) {
  return bits == 5 ? launch_regring_b5(tn, epi, a, stream) : launch_regring_b4(tn, epi, a, stream);
}

// Workspace of a K split over workgroups: fp32 partial sums, and one arrival counter per pair
// group, each zero between launches (the last workgroup of a group resets its counter).  Calls
// that share one workspace must not overlap in time.  part == nullptr: no split.
struct SplitWs {
  float* part;
  int* cnt;
  size_t part_bytes;
  int groups;
};

// 32-row register ring (regring.hip): 32x32x16 steps on tile pairs, T <= tn (32 or 64) tokens,
// any K; pairs spread evenly over one workgroup per compute unit, K optionally split
hipError_t launch_regring32_b4(int tn, int epi, const KArgs& a, const SplitWs& ws, hipStream_t stream);
hipError_t launch_regring32_b5(int tn, int epi, const KArgs& a, const SplitWs& ws, hipStream_t stream);
inline hipError_t launch_regring32(int tn, int bits, int epi, const KArgs& a, const SplitWs& ws,
                                   hipStream_t stream) {
  return bits == 5 ? launch_regring32_b5(tn, epi, a, ws, stream) : launch_regring32_b4(tn, epi, a, ws, stream);
}
// A8 route (a8.hip): int8 activations with a scale per 64 columns, and the int8 GEMM over them
// (a.x holds the int8 codes; sx the scales, [ceil(K/128)][T][2])
hipError_t launch_a8_quant(const _Float16* x, int T, int K, int8_t* xq, float* sx, hipStream_t stream);
hipError_t launch_a8(int bits, int epi, const KArgs& a, const float* sx, hipStream_t stream);
// bf16 activations [T][K] -> fp16 X[t] * 2^-e_t in xh and e_t in xexp (bf16.hip)
hipError_t launch_bf16_prep(const uint16_t* x, int T, int K, _Float16* xh, int* xexp, hipStream_t stream);
hipError_t launch_wide(int bits, int epi, const KArgs& a, hipStream_t stream);    // any T
hipError_t launch_splitk(int bits, int epi, const KArgs& a, hipStream_t stream);  // T <= 32

}  // namespace w4
