// Activation preparation for bf16 inputs.
//
// The kernels multiply fp16 activations with fp16 dequantised weights.  Every bf16 value (8
// significant bits) is exactly an fp16 value (11 significant bits) once it lies inside fp16's
// exponent range, so one power of two per token, e_t, moves a token row into that range without
// rounding: X'[t] = X[t] * 2^-e_t with e_t chosen so that the row's largest magnitude m lands in
// [2^14, 2^15) (fp16's largest finite value is 65504).  Values smaller than m * 2^-17 fall below
// fp16's 11-bit precision at that scale and are rounded (to nearest, an error below
// m * 2^-41 each); everything else is carried exactly.  The epilogues then multiply the fp32 sums
// by 2^e_t, add a bf16 residual or apply SwiGLU in fp32, and round once to bf16.
//
// Compared with dequantising to bf16 and using bf16 matrix-core steps, this keeps the weights'
// 11-bit fp16 precision and the same kernels for both activation types; the price is one small
// kernel that reads each activation row twice and writes it once in fp16 (T * K * 6 bytes).
// Rows with an infinite or NaN entry take e_t = 0, so those values propagate.
#include "device.h"
#include "kernels.h"

namespace w4 {
namespace {

using namespace w4dev;

constexpr int kThreads = 256;

// One workgroup per token row.  K is a multiple of 64, so a row is a whole number of 16-byte
// chunks of 8 values.
__global__ __launch_bounds__(kThreads) void bf16_prep_kernel(const uint16_t* __restrict__ x, int K,
                                                             _Float16* __restrict__ xh,
                                                             int* __restrict__ xexp) {
  const int t = blockIdx.x;
  const uint16_t* row = x + (size_t)t * K;
  _Float16* orow = xh + (size_t)t * K;
  const int nch = K / 8;
  // largest magnitude of the row as bits: for bf16 values that are not NaN the order of the 15
  // magnitude bits is the order of |x| (infinity, 0x7F80, sorts above every finite value)
  uint32_t m = 0;
  for (int c = threadIdx.x; c < nch; c += kThreads) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = v[e] & 0x7FFFu, hi = (v[e] >> 16) & 0x7FFFu;
      m = max(m, max(lo, hi));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  __shared__ uint32_t wmax[kThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) wmax[wave] = m;
  __syncthreads();
  m = wmax[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) m = max(m, wmax[w]);
  // e_t: m * 2^-e in [2^14, 2^15); zero rows and rows holding an infinity or NaN keep e = 0
  int e = 0;
  if (m != 0 && m < 0x7F80u) e = __builtin_amdgcn_frexp_expf(bf16_value((uint16_t)m)) - 1 - 14;
  if (threadIdx.x == 0) xexp[t] = e;
  for (int c = threadIdx.x; c < nch; c += kThreads) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * c);
    f16x8 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = (f16)ldexpf(bf16_value((uint16_t)(v[i] & 0xFFFFu)), -e);
      h[2 * i + 1] = (f16)ldexpf(bf16_value((uint16_t)(v[i] >> 16)), -e);
    }
    *reinterpret_cast<f16x8*>(orow + 8 * c) = h;
  }
}

}  // namespace

hipError_t launch_bf16_prep(const uint16_t* x, int T, int K, _Float16* xh, int* xexp,
                            hipStream_t stream) {
  if (T < 1 || K % 64) return hipErrorInvalidValue;
  return launch_kernel(&bf16_prep_kernel, dim3(T), dim3(kThreads), 0, stream, x, K, xh, xexp);
}

}  // namespace w4
