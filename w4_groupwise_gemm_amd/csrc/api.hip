// C ABI: argument validation, route table and the single launch of every compute call.
//
// Route table.  Each op has several kernels ("routes"), each with an explicit T domain; the
// public calls pick exactly one route and launch it once.  Both rules come from the failures
// the ninfer-3080 performance notes describe ("Route boundaries are measured here"): a kernel
// handed more columns than it supports corrupted memory or silently did one column's work,
// and a switch fallthrough ran a second kernel over the first.  The boundaries in
// pick_route are set from crossovers measured per route at the same T (cold weights).
#include <hip/hip_runtime.h>

#include <climits>
#include <initializer_list>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/w4gemm.h"
#include "device.h"
#include "kernels.h"
#include "layout.h"

namespace {

enum RouteKind {
  KIND_GEMV = 0,
  KIND_STREAM = 1,
  KIND_NARROW = 2,
  KIND_WIDE = 3,
  KIND_SPLITK = 4,
  KIND_STREAM32 = 5,
  KIND_STREAM64 = 6,
  KIND_BALANCED = 7,
  KIND_REGRING = 8,
  KIND_REGRING32 = 9
};

struct Route {
  const char* name;
  int tmin, tmax;
  RouteKind kind;
  int tn;  // padded token tile of the narrow routes
};

const Route kRoutes[] = {
    {"gemv_exact_t", 1, 4, KIND_GEMV, 0},
    {"mfma_stream_t16", 1, 16, KIND_STREAM, 16},
    {"mfma_narrow_t32", 1, 32, KIND_NARROW, 32},
    {"mfma_narrow_t64", 1, 64, KIND_NARROW, 64},
    {"mfma_wide", 1, INT_MAX, KIND_WIDE, 0},
    {"mfma_splitk_t32", 1, 32, KIND_SPLITK, 32},
    {"mfma_narrow_tiled", 1, INT_MAX, KIND_NARROW, 64},
    {"mfma_stream_t32", 1, 32, KIND_STREAM32, 32},
    {"mfma_stream_t64", 1, 64, KIND_STREAM64, 64},
    {"mfma_bal_t32", 1, 32, KIND_BALANCED, 32},
    {"mfma_bal_t64", 1, 64, KIND_BALANCED, 64},
    {"mfma_reg_t16", 1, 16, KIND_REGRING, 16},
    {"mfma_reg_t32", 1, 32, KIND_REGRING, 32},
    {"mfma_reg_t64", 1, 64, KIND_REGRING, 64},
    {"mfma_reg32_t32", 1, 32, KIND_REGRING32, 32},
    {"mfma_reg32_t64", 1, 64, KIND_REGRING32, 64},
};
constexpr int kNumRoutes = sizeof(kRoutes) / sizeof(kRoutes[0]);
// route ids (indices into kRoutes; R_N16 is the 16-token streaming route)
enum { R_GEMV = 0, R_N16 = 1, R_N32 = 2, R_N64 = 3, R_WIDE = 4, R_SPLITK = 5, R_NTILED = 6, R_S32 = 7,
       R_S64 = 8, R_B32 = 9, R_B64 = 10, R_R16 = 11, R_R32 = 12, R_R64 = 13, R_Q32 = 14, R_Q64 = 15 };

constexpr int kMaxDim = 1 << 24;

bool op_ok(int op) { return op == W4_OP_LINEAR || op == W4_OP_SWIGLU || op == W4_OP_ADD; }

// Shape-only checks shared by validation and route selection (no pointers, no HIP calls).
int check_shape(int op, int T, int N, int K, int bits, int group) {
  if (!op_ok(op)) return W4_ERR_UNSUPPORTED;
  if (bits != 4 && bits != 5) return W4_ERR_UNSUPPORTED;
  if (!w4layout::group_ok(group)) return W4_ERR_UNSUPPORTED;
  if (T < 0 || N <= 0 || K <= 0) return W4_ERR_INVALID_ARG;
  if (T > kMaxDim || N > kMaxDim || K > kMaxDim) return W4_ERR_INVALID_ARG;
  if (N % w4layout::kRowTile || K % w4layout::k_multiple(group)) return W4_ERR_INVALID_ARG;
  return W4_OK;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// x_optional: x may be NULL (the A8 calls with pre-quantised activations); it is then not checked.
int validate(int op, const void* x, const void* w, const void* s, const void* z, const void* res,
             int T, int N, int K, int bits, int group, const void* out, bool x_optional = false) {
  int st = check_shape(op, T, N, K, bits, group);
  if (st != W4_OK) return st;
  if (T == 0) return W4_OK;
  if ((!x && !x_optional) || !w || !s || !z || !out) return W4_ERR_INVALID_ARG;
  if (op == W4_OP_ADD && !res) return W4_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(s) || !aligned16(z) || !aligned16(out))
    return W4_ERR_MISALIGNED;
  if (op == W4_OP_ADD && !aligned16(res)) return W4_ERR_MISALIGNED;
  const int rows = op == W4_OP_SWIGLU ? 2 * N : N;
  const size_t wbytes = w4_packed_bytes(rows, K, bits, group);
  const size_t szbytes = w4_packed_sz_bytes(rows, K, group);
  auto rng = [](const void* p, size_t n) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return Range{b, b + n};
  };
  // 32-bit buffer offsets: every tensor must stay below 2 GiB
  const size_t kLimit = (size_t)1 << 31;
  if ((size_t)T * K * 2 >= kLimit || (size_t)T * N * 2 >= kLimit || wbytes >= kLimit)
    return W4_ERR_UNSUPPORTED;
  const Range ro = rng(out, (size_t)T * N * 2);
  if ((x && overlap(ro, rng(x, (size_t)T * K * 2))) || overlap(ro, rng(w, wbytes)) ||
      overlap(ro, rng(s, szbytes)) || overlap(ro, rng(z, szbytes)))
    return W4_ERR_ALIAS;
  if (op == W4_OP_ADD && res != out && overlap(ro, rng(res, (size_t)T * N * 2)))
    return W4_ERR_ALIAS;
  return W4_OK;
}

// Per-device "is gfx950" cache: 0 unknown, 1 yes, -1 no.  Filled once per device by a host
// property query (no stream work), so the hot path stays capturable.
int g_arch_ok[64];

int device_check() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return W4_ERR_DEVICE;
  if (dev >= 64) return W4_ERR_DEVICE;
  int v = __atomic_load_n(&g_arch_ok[dev], __ATOMIC_ACQUIRE);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return W4_ERR_DEVICE;
    v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    __atomic_store_n(&g_arch_ok[dev], v, __ATOMIC_RELEASE);
  }
  return v == 1 ? W4_OK : W4_ERR_DEVICE;
}

// Boundaries from route sweeps on this chip (every route timed at the same T, cold weights, at
// the decode, batched-decode, SwiGLU-pair and 5120-row prefill shapes and at 5120-row matrices
// of K = 8192 .. 17408); the reasons are given case by case below.
int pick_route(int op, int bits, int T, int N, int K) {
  // Crossovers measured per route on cold weights (us per launch):
  //  * K <= 5120, single matrices: the streaming route holds each wave's activation slice in LDS
  //    and leads to 16 tokens, its 32-row ring to 32 and its 64-row ring to 64 with 4-bit codes
  //    (12288 x 5120, T = 16 / 32 / 64: 11.1 / 12.4 / 18.7 against 12.4 / 16.1 / 25.7 for the
  //    register ring).  With 5-bit codes (more vector work per code byte) the register ring
  //    leads at 5-16 tokens (12288 rows, T = 8: 11.7 against 13.2) and at 33-48 (T = 33 / 48:
  //    19.0 / 22.3 against 21.5 / 22.5 narrow), the narrow kernel beyond.
  //  * The SwiGLU pair at K <= 5120 depends on the pairs per compute unit.  One or fewer (4096
  //    rows): the streaming routes throughout (T = 16 / 32 / 64: 8.7 / 10.1 / 14.7 against 10.3 /
  //    14.9 / 24.2 register ring, 13.1 / 13.4 / 17.4 evenly spread narrow).  More: the streaming
  //    route to 8 tokens (17408 rows, T = 8: 25.9 against 27.2), then the register ring, whose
  //    32-token instance already leads at 9-16 tokens when a compute unit holds three or more
  //    pairs (17408 rows, T = 16 / 32 / 64: 27.2 / 28.8 / 39.1 against 31.6 / 31.6 / 47.1 evenly
  //    spread narrow); with two (5-bit 8192 rows) its 16-token instance to 16 (15.8 against
  //    17.7 streamed), and the evenly spread narrow kernel above 48 (T = 64: 25.8 against 27.7).
  //  * K > 5120, single matrices (5120 rows, K = 6144 .. 17408): the 32-row register ring, with
  //    K split three ways over the workgroups from K = 8192, leads from 17 tokens, from 13 once
  //    K >= 12288 and from the first token once K > 16384 (4-bit 17408 columns, T = 1 / 16 / 32
  //    / 64: 18.6 / 19.5 / 19.5 / 28.6 against 19.4 / 22.7 16-row ring, 31.9 / 43.0 narrow;
  //    5-bit 6144 columns, unsplit, T = 24 / 64: 12.9 / 18.9 against 14.5 / 19.9 before it).
  //    Below, the 16-row register ring from 5 tokens, and from the first token once K > 8192
  //    (5-bit 12288 columns, T = 1: 16.8 against 17.4 32-row ring); streaming at 1-4 tokens up
  //    to K = 8192 (4-bit 8192 columns, T = 1: 9.3 against 10.9).
  //  * The SwiGLU pair at K > 5120 has no measured shape (the pair's workloads all have
  //    K = 5120); it keeps the order measured before the register ring existed.
  if (K <= 5120) {
    if (op == W4_OP_SWIGLU) {
      const int pairs = N / 16;
      if (pairs <= 256) {
        if (T <= 16) return R_N16;
        if (T <= 32) return R_S32;
        if (T <= 64) return R_S64;
      } else {
        if (T <= 8) return R_N16;
        if (pairs >= 3 * 256) {
          if (T <= 32) return R_R32;
          if (T <= 64) return R_R64;
        } else {
          if (T <= 16) return R_R16;
          if (T <= 32) return R_R32;
          if (T <= 48) return R_R64;
          if (T <= 64) return R_B64;
        }
      }
    } else if (bits == 5) {
      if (T <= 4) return R_N16;
      if (T <= 16) return R_R16;
      if (T <= 32) return R_S32;
      if (T <= 48) return R_R64;
      if (T <= 64) return R_N64;
    } else {
      if (T <= 16) return R_N16;
      if (T <= 32) return R_S32;
      if (T <= 64) return R_S64;
    }
  } else if (op == W4_OP_SWIGLU) {
    if (T <= 16) return R_N16;
    if (T <= 32) return R_N32;
    if (T <= 64) return R_N64;
  } else {
    if (K > 16384 && T <= 32) return R_Q32;
    if (T <= 4) return K > 8192 ? R_R16 : R_N16;
    if (T <= 12) return R_R16;
    if (T <= 16) return K >= 12288 ? R_Q32 : R_R16;
    if (T <= 32) return R_Q32;
    if (T <= 64) return R_Q64;
  }
  // Above 64 tokens the wide kernel's workgroups (about 128 rows x 128 tokens each) leave most
  // compute units idle until there are about 128 of them; below that the narrow kernel run as
  // side-by-side 64-token blocks is faster (5120 rows: 34 vs 73 us at T = 128, 67 vs 73 at 384,
  // 81 vs 74 at 512; 11264 rows: 36 vs 46 at 128, 54 vs 47 at 256).
  const long long rows = op == W4_OP_SWIGLU ? 2LL * N : (long long)N;
  if ((rows + 127) / 128 * ((T + 127) / 128) < 128) return R_NTILED;
  return R_WIDE;
}

// ---- Workspace of the K split over workgroups (32-row register ring): static device arrays, one
// slot per stream (calls on one stream never overlap; calls on different streams get different
// slots).  Each slot's counters start at zero and every launch leaves them at zero.  A stream
// beyond the last slot runs the routes without the split.
constexpr int kSplitSlots = 4;
constexpr size_t kSplitBytes = (size_t)8 << 20;
constexpr int kSplitGroups = 256;
__device__ __align__(256) float split_part[kSplitSlots][kSplitBytes / 4];
__device__ __align__(256) int split_cnt[kSplitSlots][kSplitGroups] = {};

struct SplitSlots {
  char* part = nullptr;
  int* cnt = nullptr;
  hipStream_t owner[kSplitSlots] = {};
  bool used[kSplitSlots] = {};
};
SplitSlots g_split[64];
std::mutex g_split_mu;

w4::SplitWs split_ws_for(hipStream_t st) {
  w4::SplitWs none{nullptr, nullptr, 0, 0};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return none;
  std::lock_guard<std::mutex> lock(g_split_mu);
  SplitSlots& d = g_split[dev];
  if (!d.part) {
    void* p = nullptr;
    void* c = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(split_part)) != hipSuccess || !p) return none;
    if (hipGetSymbolAddress(&c, HIP_SYMBOL(split_cnt)) != hipSuccess || !c) return none;
    d.part = static_cast<char*>(p);
    d.cnt = static_cast<int*>(c);
  }
  int slot = -1;
  for (int i = 0; i < kSplitSlots && slot < 0; ++i)
    if (d.used[i] && d.owner[i] == st) slot = i;
  for (int i = 0; i < kSplitSlots && slot < 0; ++i)
    if (!d.used[i]) {
      d.used[i] = true;
      d.owner[i] = st;
      slot = i;
    }
  if (slot < 0) return none;
  return w4::SplitWs{reinterpret_cast<float*>(d.part + slot * kSplitBytes), d.cnt + slot * kSplitGroups,
                     kSplitBytes, kSplitGroups};
}

// xexp: nullptr for fp16 activations and outputs; for bf16 ones, x is the prepared fp16 copy and
// xexp its per-token exponents (outputs and residual are then bf16).
int launch_route(int route, int op, const void* x, const void* w, const void* s, const void* z,
                 const void* res, int T, int N, int K, int bits, int group, void* out,
                 void* stream, const int* xexp = nullptr) {
  const Route& R = kRoutes[route];
  if (T < R.tmin || T > R.tmax) return W4_ERR_DOMAIN;
  w4::KArgs a;
  a.x = static_cast<const _Float16*>(x);
  a.w = static_cast<const uint8_t*>(w);
  a.sc = static_cast<const uint32_t*>(s);
  a.zr = static_cast<const uint32_t*>(z);
  a.res = op == W4_OP_ADD ? static_cast<const _Float16*>(res) : nullptr;
  a.out = static_cast<_Float16*>(out);
  a.T = T;
  a.rows = op == W4_OP_SWIGLU ? 2 * N : N;
  a.K = K;
  a.KB = w4layout::num_kblocks(K);
  a.ldo = N;
  a.szw = w4layout::sz_words(group);
  a.xexp = xexp;
  const int epi = op == W4_OP_SWIGLU ? w4dev::EPI_SWIGLU
                  : op == W4_OP_ADD  ? w4dev::EPI_ADD
                                     : w4dev::EPI_STORE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (R.kind) {
    case KIND_GEMV: e = w4::launch_gemv(bits, epi, a, st); break;
    case KIND_STREAM: e = w4::launch_stream16(bits, epi, a, st); break;
    case KIND_NARROW: e = w4::launch_narrow(R.tn, false, bits, epi, a, st); break;
    case KIND_BALANCED: e = w4::launch_narrow(R.tn, true, bits, epi, a, st); break;
    case KIND_REGRING: e = w4::launch_regring(R.tn, bits, epi, a, st); break;
    case KIND_REGRING32: e = w4::launch_regring32(R.tn, bits, epi, a, split_ws_for(st), st); break;
    case KIND_WIDE: e = w4::launch_wide(bits, epi, a, st); break;
    case KIND_SPLITK: e = w4::launch_splitk(bits, epi, a, st); break;
    case KIND_STREAM32:
      // the 32-row activation ring of the streaming kernel covers K <= 5120 (five k-blocks per
      // wave); longer rows run this route's schedule on the narrow kernel's 32-token tile
      e = K <= 5120 ? w4::launch_stream32(bits, epi, a, st) : w4::launch_narrow(32, false, bits, epi, a, st);
      break;
    case KIND_STREAM64:  // likewise with 64-row tiles
      e = K <= 5120 ? w4::launch_stream64(bits, epi, a, st) : w4::launch_narrow(64, false, bits, epi, a, st);
      break;
    default: return W4_ERR_DOMAIN;
  }
  return e == hipSuccess ? W4_OK : W4_ERR_LAUNCH;
}

int run_op(int route, int op, const void* x, const void* w, const void* s, const void* z,
           const void* res, int T, int N, int K, int bits, int group, void* out, void* stream) {
  int st = validate(op, x, w, s, z, res, T, N, K, bits, group, out);
  if (st != W4_OK) return st;
  if (route < 0) route = pick_route(op, bits, T, N, K);
  if (route >= kNumRoutes) return W4_ERR_DOMAIN;
  if (T == 0) return W4_OK;
  if (T < kRoutes[route].tmin || T > kRoutes[route].tmax) return W4_ERR_DOMAIN;
  st = device_check();
  if (st != W4_OK) return st;
  return launch_route(route, op, x, w, s, z, res, T, N, K, bits, group, out, stream);
}

constexpr size_t align16(size_t n) { return (n + 15) & ~(size_t)15; }

// Workspace of a bf16 call: the fp16 copy of X (T x K) and the T per-token exponents.
size_t bf16_ws_bytes(int T, int K) { return align16((size_t)T * K * 2) + align16((size_t)T * 4); }

// bf16 activations: validate as the fp16 op (the tensors have the same sizes) plus the workspace,
// then enqueue the preparation kernel (X[t] * 2^-e_t in fp16, and e_t) and the route's kernel.
int run_op_bf16(int route, int op, const void* x, const void* w, const void* s, const void* z,
                const void* res, int T, int N, int K, int bits, int group, void* out, void* ws,
                size_t ws_bytes, void* stream) {
  int st = validate(op, x, w, s, z, res, T, N, K, bits, group, out);
  if (st != W4_OK) return st;
  if (route < 0) route = pick_route(op, bits, T, N, K);
  if (route >= kNumRoutes) return W4_ERR_DOMAIN;
  if (T == 0) return W4_OK;
  if (T < kRoutes[route].tmin || T > kRoutes[route].tmax) return W4_ERR_DOMAIN;
  if (!ws) return W4_ERR_INVALID_ARG;
  if (!aligned16(ws)) return W4_ERR_MISALIGNED;
  const size_t need = bf16_ws_bytes(T, K);
  if (ws_bytes < need) return W4_ERR_INVALID_ARG;
  const int rows = op == W4_OP_SWIGLU ? 2 * N : N;
  auto rng = [](const void* p, size_t n) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return Range{b, b + n};
  };
  const Range rw = rng(ws, need);
  if (overlap(rw, rng(x, (size_t)T * K * 2)) || overlap(rw, rng(out, (size_t)T * N * 2)) ||
      overlap(rw, rng(w, w4_packed_bytes(rows, K, bits, group))) ||
      overlap(rw, rng(s, w4_packed_sz_bytes(rows, K, group))) ||
      overlap(rw, rng(z, w4_packed_sz_bytes(rows, K, group))) ||
      (op == W4_OP_ADD && overlap(rw, rng(res, (size_t)T * N * 2))))
    return W4_ERR_ALIAS;
  st = device_check();
  if (st != W4_OK) return st;
  _Float16* xh = static_cast<_Float16*>(ws);
  int* xexp = reinterpret_cast<int*>(static_cast<char*>(ws) + align16((size_t)T * K * 2));
  if (w4::launch_bf16_prep(static_cast<const uint16_t*>(x), T, K, xh, xexp,
                           static_cast<hipStream_t>(stream)) != hipSuccess)
    return W4_ERR_LAUNCH;
  return launch_route(route, op, xh, w, s, z, res, T, N, K, bits, group, out, stream, xexp);
}

}  // namespace

extern "C" int w4_linear(const uint16_t* x, const void* w, const uint16_t* scales,
                         const uint16_t* zeros, int T, int N, int K, int bits, int group,
                         uint16_t* out, void* stream) {
  return run_op(-1, W4_OP_LINEAR, x, w, scales, zeros, nullptr, T, N, K, bits, group, out, stream);
}

extern "C" int w4_linear_swiglu(const uint16_t* x, const void* w_pair,
                                const uint16_t* scales_pair, const uint16_t* zeros_pair, int T,
                                int N, int K, int bits, int group, uint16_t* out, void* stream) {
  return run_op(-1, W4_OP_SWIGLU, x, w_pair, scales_pair, zeros_pair, nullptr, T, N, K, bits,
                group, out, stream);
}

extern "C" int w4_linear_add(const uint16_t* x, const void* w, const uint16_t* scales,
                             const uint16_t* zeros, const uint16_t* residual, int T, int N, int K,
                             int bits, int group, uint16_t* out, void* stream) {
  return run_op(-1, W4_OP_ADD, x, w, scales, zeros, residual, T, N, K, bits, group, out, stream);
}

extern "C" int w4_linear_grouped(const uint16_t* x, const w4_parent* parents, int nparents, int T,
                                 int K, int group, void* stream) {
  if (!parents || nparents < 1 || nparents > W4_MAX_PARENTS) return W4_ERR_INVALID_ARG;
  static_assert(W4_MAX_PARENTS == w4::kMaxParents, "one limit");
  for (int p = 0; p < nparents; ++p) {
    const w4_parent& q = parents[p];
    const int st = validate(W4_OP_LINEAR, x, q.w, q.scales, q.zeros, nullptr, T, q.N, K, q.bits,
                            group, q.out);
    if (st != W4_OK) return st;
  }
  if (T == 0) return W4_OK;
  // no output may overlap another matrix's output or inputs
  auto rng = [](const void* ptr, size_t n) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(ptr);
    return Range{b, b + n};
  };
  for (int p = 0; p < nparents; ++p) {
    const Range ro = rng(parents[p].out, (size_t)T * parents[p].N * 2);
    for (int q = 0; q < nparents; ++q) {
      if (q == p) continue;
      const w4_parent& o = parents[q];
      const size_t szb = w4_packed_sz_bytes(o.N, K, group);
      if (overlap(ro, rng(o.out, (size_t)T * o.N * 2)) || overlap(ro, rng(o.w, w4_packed_bytes(o.N, K, o.bits, group))) ||
          overlap(ro, rng(o.scales, szb)) || overlap(ro, rng(o.zeros, szb)))
        return W4_ERR_ALIAS;
    }
  }
  const int st = device_check();
  if (st != W4_OK) return st;
  if (T <= 64 && K <= 5120) {
    w4::GroupedArgs g;
    g.n = nparents;
    for (int p = 0; p < nparents; ++p) {
      w4::KArgs& a = g.a[p];
      a.x = reinterpret_cast<const _Float16*>(x);
      a.w = static_cast<const uint8_t*>(parents[p].w);
      a.sc = reinterpret_cast<const uint32_t*>(parents[p].scales);
      a.zr = reinterpret_cast<const uint32_t*>(parents[p].zeros);
      a.res = nullptr;
      a.out = reinterpret_cast<_Float16*>(parents[p].out);
      a.T = T;
      a.rows = parents[p].N;
      a.K = K;
      a.KB = w4layout::num_kblocks(K);
      a.ldo = parents[p].N;
      a.szw = w4layout::sz_words(group);
      a.xexp = nullptr;
      g.bits[p] = parents[p].bits;
    }
    return w4::launch_grouped(g, static_cast<hipStream_t>(stream)) == hipSuccess ? W4_OK : W4_ERR_LAUNCH;
  }
  for (int p = 0; p < nparents; ++p) {
    const w4_parent& q = parents[p];
    const int e = launch_route(pick_route(W4_OP_LINEAR, q.bits, T, q.N, K), W4_OP_LINEAR, x, q.w, q.scales,
                               q.zeros, nullptr, T, q.N, K, q.bits, group, q.out, stream);
    if (e != W4_OK) return e;
  }
  return W4_OK;
}

// ---- A8 route: int8 activations (scale per 64 columns), int8 matrix-core GEMM
size_t a8_ws_bytes(int T, int K) {
  return align16((size_t)T * K) + (size_t)w4layout::num_kblocks(K) * T * 2 * sizeof(float);
}

// Workspace checks shared by the A8 calls: present, aligned, large enough, overlapping none of
// the given ranges.
int check_a8_ws(const void* ws, size_t ws_bytes, int T, int K, std::initializer_list<Range> others) {
  if (!ws) return W4_ERR_INVALID_ARG;
  if (!aligned16(ws)) return W4_ERR_MISALIGNED;
  const size_t need = a8_ws_bytes(T, K);
  if (ws_bytes < need) return W4_ERR_INVALID_ARG;
  const uintptr_t b = reinterpret_cast<uintptr_t>(ws);
  for (const Range& r : others)
    if (overlap(Range{b, b + need}, r)) return W4_ERR_ALIAS;
  return W4_OK;
}

Range span(const void* p, size_t n) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  return Range{b, b + (p ? n : 0)};
}

int run_a8(int op, const void* x, const void* w, const void* s, const void* z, const void* res, int T,
           int N, int K, int bits, int group, void* out, void* ws, size_t ws_bytes, void* stream) {
  if (group != 64) return check_shape(op, T, N, K, bits, group) == W4_OK ? W4_ERR_UNSUPPORTED
                                                                          : check_shape(op, T, N, K, bits, group);
  // x may be NULL: the workspace then already holds this T x K activation, quantised by
  // w4_quantize_a8
  int st = validate(op, x, w, s, z, res, T, N, K, bits, group, out, /*x_optional=*/true);
  if (st != W4_OK) return st;
  if (T == 0) return W4_OK;
  const int rows = op == W4_OP_SWIGLU ? 2 * N : N;
  st = check_a8_ws(ws, ws_bytes, T, K,
                   {span(x, (size_t)T * K * 2), span(out, (size_t)T * N * 2),
                    span(w, w4_packed_bytes(rows, K, bits, group)), span(s, w4_packed_sz_bytes(rows, K, group)),
                    span(z, w4_packed_sz_bytes(rows, K, group)),
                    span(op == W4_OP_ADD ? res : nullptr, (size_t)T * N * 2)});
  if (st != W4_OK) return st;
  st = device_check();
  if (st != W4_OK) return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  int8_t* xq = static_cast<int8_t*>(ws);
  float* sx = reinterpret_cast<float*>(static_cast<char*>(ws) + align16((size_t)T * K));
  if (x && w4::launch_a8_quant(static_cast<const _Float16*>(x), T, K, xq, sx, hs) != hipSuccess)
    return W4_ERR_LAUNCH;
  w4::KArgs a;
  a.x = reinterpret_cast<const _Float16*>(xq);
  a.w = static_cast<const uint8_t*>(w);
  a.sc = static_cast<const uint32_t*>(s);
  a.zr = static_cast<const uint32_t*>(z);
  a.res = op == W4_OP_ADD ? static_cast<const _Float16*>(res) : nullptr;
  a.out = static_cast<_Float16*>(out);
  a.T = T;
  a.rows = rows;
  a.K = K;
  a.KB = w4layout::num_kblocks(K);
  a.ldo = N;
  a.szw = w4layout::sz_words(group);
  a.xexp = nullptr;
  const int epi = op == W4_OP_SWIGLU ? w4dev::EPI_SWIGLU : op == W4_OP_ADD ? w4dev::EPI_ADD : w4dev::EPI_STORE;
  return w4::launch_a8(bits, epi, a, sx, hs) == hipSuccess ? W4_OK : W4_ERR_LAUNCH;
}

extern "C" size_t w4_a8_workspace_bytes(int T, int K) {
  if (T < 0 || K <= 0 || T > kMaxDim || K > kMaxDim || K % 64) return 0;
  return a8_ws_bytes(T, K);
}

extern "C" int w4_quantize_a8(const uint16_t* x, int T, int K, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (T < 0 || K <= 0 || T > kMaxDim || K > kMaxDim || K % 64) return W4_ERR_INVALID_ARG;
  if (T == 0) return W4_OK;
  if (!x) return W4_ERR_INVALID_ARG;
  if (!aligned16(x)) return W4_ERR_MISALIGNED;
  int st = check_a8_ws(workspace, workspace_bytes, T, K, {span(x, (size_t)T * K * 2)});
  if (st != W4_OK) return st;
  st = device_check();
  if (st != W4_OK) return st;
  int8_t* xq = static_cast<int8_t*>(workspace);
  float* sx = reinterpret_cast<float*>(static_cast<char*>(workspace) + align16((size_t)T * K));
  return w4::launch_a8_quant(reinterpret_cast<const _Float16*>(x), T, K, xq, sx,
                             static_cast<hipStream_t>(stream)) == hipSuccess ? W4_OK : W4_ERR_LAUNCH;
}

extern "C" int w4_linear_a8(const uint16_t* x, const void* w, const uint16_t* scales, const uint16_t* zeros,
                            int T, int N, int K, int bits, int group, uint16_t* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return run_a8(W4_OP_LINEAR, x, w, scales, zeros, nullptr, T, N, K, bits, group, out, workspace,
                workspace_bytes, stream);
}

extern "C" int w4_linear_swiglu_a8(const uint16_t* x, const void* w_pair, const uint16_t* scales_pair,
                                   const uint16_t* zeros_pair, int T, int N, int K, int bits, int group,
                                   uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  return run_a8(W4_OP_SWIGLU, x, w_pair, scales_pair, zeros_pair, nullptr, T, N, K, bits, group, out,
                workspace, workspace_bytes, stream);
}

extern "C" int w4_linear_add_a8(const uint16_t* x, const void* w, const uint16_t* scales,
                                const uint16_t* zeros, const uint16_t* residual, int T, int N, int K,
                                int bits, int group, uint16_t* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return run_a8(W4_OP_ADD, x, w, scales, zeros, residual, T, N, K, bits, group, out, workspace,
                workspace_bytes, stream);
}

extern "C" size_t w4_bf16_workspace_bytes(int T, int K) {
  if (T < 0 || K <= 0 || T > kMaxDim || K > kMaxDim || K % 64) return 0;
  return bf16_ws_bytes(T, K);
}

extern "C" int w4_linear_bf16(const uint16_t* x, const void* w, const uint16_t* scales,
                              const uint16_t* zeros, int T, int N, int K, int bits, int group,
                              uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  return run_op_bf16(-1, W4_OP_LINEAR, x, w, scales, zeros, nullptr, T, N, K, bits, group, out,
                     workspace, workspace_bytes, stream);
}

extern "C" int w4_linear_swiglu_bf16(const uint16_t* x, const void* w_pair,
                                     const uint16_t* scales_pair, const uint16_t* zeros_pair, int T,
                                     int N, int K, int bits, int group, uint16_t* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return run_op_bf16(-1, W4_OP_SWIGLU, x, w_pair, scales_pair, zeros_pair, nullptr, T, N, K, bits,
                     group, out, workspace, workspace_bytes, stream);
}

extern "C" int w4_linear_add_bf16(const uint16_t* x, const void* w, const uint16_t* scales,
                                  const uint16_t* zeros, const uint16_t* residual, int T, int N,
                                  int K, int bits, int group, uint16_t* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return run_op_bf16(-1, W4_OP_ADD, x, w, scales, zeros, residual, T, N, K, bits, group, out,
                     workspace, workspace_bytes, stream);
}

// ---- allocation-free bf16 linear: the workspace is this file's static device array.  The host
// name `scratch` is only a stand-in for the device symbol; its device address is looked up
// once per device (with that device current) and kept, and only that address is ever handed
// to a kernel.
namespace {
__device__ __align__(256) char scratch[W4_SCRATCH_BYTES];

void* g_scratch_ptr[64];
std::mutex g_scratch_mu;

int scratch_for_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return W4_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return W4_ERR_SCRATCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return W4_OK;
}
}  // namespace

extern "C" int w4_linear_bf16_noalloc(const uint16_t* x, const void* w, const uint16_t* scales,
                                      const uint16_t* zeros, int T, int N, int K, int bits,
                                      int group, uint16_t* out, void* stream) {
  int st = check_shape(W4_OP_LINEAR, T, N, K, bits, group);
  if (st != W4_OK) return st;
  if (T == 0) return W4_OK;
  if (bf16_ws_bytes(T, K) > (size_t)W4_SCRATCH_BYTES) return W4_ERR_SCRATCH;
  st = device_check();
  if (st != W4_OK) return st;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != W4_OK) return st;
  return run_op_bf16(-1, W4_OP_LINEAR, x, w, scales, zeros, nullptr, T, N, K, bits, group, out, ws,
                     W4_SCRATCH_BYTES, stream);
}

extern "C" int w4_linear_route_bf16(int route_id, int op, const uint16_t* x, const void* w,
                                    const uint16_t* scales, const uint16_t* zeros,
                                    const uint16_t* residual, int T, int N, int K, int bits,
                                    int group, uint16_t* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (route_id < 0 || route_id >= kNumRoutes) return W4_ERR_DOMAIN;
  return run_op_bf16(route_id, op, x, w, scales, zeros, residual, T, N, K, bits, group, out,
                     workspace, workspace_bytes, stream);
}

extern "C" int w4_route_for(int op, int bits, int T, int N, int K) {
  int st = check_shape(op, T, N, K, bits, w4layout::kGroup);
  if (st != W4_OK) return st;
  return pick_route(op, bits, T < 1 ? 1 : T, N, K);
}

extern "C" int w4_linear_route(int route_id, int op, const uint16_t* x, const void* w,
                               const uint16_t* scales, const uint16_t* zeros,
                               const uint16_t* residual, int T, int N, int K, int bits, int group,
                               uint16_t* out, void* stream) {
  if (route_id < 0 || route_id >= kNumRoutes) return W4_ERR_DOMAIN;
  return run_op(route_id, op, x, w, scales, zeros, residual, T, N, K, bits, group, out, stream);
}

extern "C" int w4_route_count(void) { return kNumRoutes; }

extern "C" const char* w4_route_name(int route_id) {
  if (route_id < 0 || route_id >= kNumRoutes) return nullptr;
  return kRoutes[route_id].name;
}

extern "C" int w4_route_domain(int route_id, int* tmin, int* tmax) {
  if (route_id < 0 || route_id >= kNumRoutes) return W4_ERR_DOMAIN;
  if (tmin) *tmin = kRoutes[route_id].tmin;
  if (tmax) *tmax = kRoutes[route_id].tmax;
  return W4_OK;
}

extern "C" const char* w4_status_str(int status) {
  switch (status) {
    case W4_OK: return "ok";
    case W4_ERR_INVALID_ARG: return "invalid argument";
    case W4_ERR_UNSUPPORTED: return "unsupported bits, group or op";
    case W4_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case W4_ERR_ALIAS: return "output overlaps an input";
    case W4_ERR_DOMAIN: return "route unknown or T outside its domain";
    case W4_ERR_DEVICE: return "no gfx950 device current";
    case W4_ERR_LAUNCH: return "kernel launch failed";
    case W4_ERR_SCRATCH: return "static scratch too small or not found on this device";
    default: return "unknown status";
  }
}

extern "C" int w4_layout_version(void) { return W4_LAYOUT_VERSION; }
