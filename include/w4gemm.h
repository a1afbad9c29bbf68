/*
 * w4gemm.h -- C ABI of the groupwise low-bit dequantize + matrix multiply library
 * for AMD Instinct MI355X (gfx950).
 *
 *   Y[T, N] = X[T, K] . dequant(Wq)[N, K]^T,   dequant(Wq)[n, k] = s[n, g] * (q[n, k] - z[n, g]),
 *   g = k / group,  q in [0, 2^bits),  bits in {4, 5},  group in {32, 64, 128} (64 measured).
 *
 * Sources.  The operation is the fused kernel of ARK research "Fused kernels" (section "Why
 * standard kernels stall": unpack the low-bit weights and multiply in one pass shaped for a
 * batch) and of the ninfer-3080 performance notes (sections "What changed" and "A8 prefill
 * routes": Q4/Q5 groupwise projections, the gate_up SwiGLU pair and the LinearAdd op, one
 * scale per 64 columns per the "cuBLAS prefill route" section).  The pages give no zero-point
 * rule, no dtype for activations and no signature; this library reads them as: zero-point z
 * in code units (w = s * (q - z)), fp16 activations/scales/zero-points/outputs, fp32
 * accumulation, one round-to-nearest-even rounding of each output.
 *
 * Conventions shared by every entry point:
 *   - fp16 tensors are passed as uint16_t bit patterns.
 *   - Device pointers are owned by the caller; the library never allocates, frees or keeps
 *     them.  Host pointers (repack) are likewise the caller's.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Compute calls validate every
 *     argument synchronously first, then enqueue exactly one kernel on `stream` (the bf16 calls:
 *     two) and return without synchronising: they are asynchronous and may be captured into a
 *     HIP graph.
 *   - On any error the call returns a negative w4_status before touching device memory;
 *     `out` is left untouched.  W4_ERR_LAUNCH is the status of this call's own kernel launch
 *     (hipLaunchKernel's return value), not an error left pending by earlier work.
 *   - The library is stateless apart from a per-device "is gfx950" cache, so concurrent calls
 *     on different streams are safe.
 */
#ifndef W4GEMM_H
#define W4GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4_LAYOUT_VERSION 1

typedef enum {
  W4_OK = 0,
  W4_ERR_INVALID_ARG = -1, /* null pointer, negative or zero size, N % 16 or K % 64 not 0
                              (K % 128 for groups of 128), workspace too small              */
  W4_ERR_UNSUPPORTED = -2, /* bits not in {4,5}, group not in {32,64,128}, unknown op       */
  W4_ERR_MISALIGNED = -3,  /* a pointer is not 16-byte aligned                              */
  W4_ERR_ALIAS = -4,       /* out overlaps an input (out == residual exactly is allowed)    */
  W4_ERR_DOMAIN = -5,      /* route forced outside its T domain, or route id unknown        */
  W4_ERR_DEVICE = -6,      /* current device is not gfx950, or no device                    */
  W4_ERR_LAUNCH = -7,      /* the kernel launch failed                                       */
  W4_ERR_SCRATCH = -8      /* the allocation-free call needs more than its static scratch,
                              or the scratch could not be located on the current device      */
} w4_status;

/* op codes for w4_route_for / w4_linear_route */
#define W4_OP_LINEAR 0
#define W4_OP_SWIGLU 1
#define W4_OP_ADD 2

/* ------------------------------------------------------------------------------------------
 * Canonical (user-side) weight format -- what w4_repack reads.
 *   4-bit: lo  uint8 [N][K/2]; code(n,k) = (lo[n][k/2] >> (4*(k&1))) & 0xF (even k = low nibble)
 *   5-bit: lo as above holds bits 0..3; hi uint8 [N][K/8] holds bit 4:
 *          (hi[n][k/8] >> (k&7)) & 1  (the 4-bit plane + high-bit plane of the ninfer-3080
 *          performance notes, "What changed", Q5 bullet).
 *   scales, zeros: fp16 [N][K/group].  The pages use one scale per 64 columns (ninfer-3080
 *   performance notes, "cuBLAS prefill route"); groups of 32 and 128 are variants.
 *
 * Packed (device) layout -- what the compute calls read.  Row tiles of 16 rows, k-blocks of
 * 128 columns, KB = ceil(K/128).  Byte image of one (row tile rt, k-block kb) block:
 *   4-bit: 1024 B = 64 lanes x 16 B.      5-bit: 1280 B = 64 lanes x 16 B (low plane), then
 *                                                 64 lanes x 4 B (high plane).
 *   blocks are stored rt-major: offset = (rt * KB + kb) * block_bytes.
 *   Lane l serves row 16*rt + (l % 16); its lane group is g = l / 16.  Dword j (0..3) of the
 *   lane's 16 low-plane bytes holds 8 codes, slots e = 0..7, for
 *       k = 128*kb + 64*(j>>1) + 16*g + 8*(j&1) + e,
 *   slot e in bits [4*(e>>1) + 16*(e&1), +4).  Dwords 0,1 lie in group 2*kb and 2,3 in group
 *   2*kb+1, so every 32-k matrix-core step stays inside one group; inside a group the k order
 *   is permuted, which leaves the product unchanged when activations follow the same order
 *   (ninfer-3080 performance notes, "What changed", "Permuted k order").
 *   5-bit high plane: the lane's 32-bit word holds bit 4 of slot e of dword j at bit
 *       t_j + r_e,  t = {0, 2, 8, 10},  r = {0, 16, 4, 20, 1, 17, 5, 21}.
 *   scales / zeros, group 64: fp16 [N/16][KB][16][2]; element (rt, kb, r, h) = value of row
 *   16*rt + r, group 2*kb + h (the group of the lane's dwords 2h, 2h+1).
 *   group 32: fp16 [N/16][KB][2][16][2]; element (rt, kb, p, r, h) = group 4*kb + 2*h + p of
 *   row 16*rt + r (the group of dwords 2h, 2h+1 of lane groups g = 2p, 2p+1).
 *   group 128: as group 64 with both halves of a pair equal to group kb (the kernels read every
 *   group size as pairs; this costs N*K/64 bytes of scales and zeros, twice the minimum).
 *   When K % 128 == 64 the second half of the last k-block is padding: codes 0, and its scale
 *   and zero entries 0.  Repacking is a bit-exact permutation plus that zero padding (and, for
 *   groups of 128, the duplicated pair halves).
 *   The packed form of a row-concatenation [A; B] (same K, bits) is the byte concatenation of
 *   the packed forms of A and B, so parents that share one activation can be packed into one
 *   buffer and run as one call.
 *   SwiGLU pair layout (w4_repack_pair): packed row tile 2i = gate rows 16i..16i+15 and
 *   packed row tile 2i+1 = up rows 16i..16i+15, i.e. a packed matrix of 2N rows.
 * ---------------------------------------------------------------------------------------- */

/* Bytes of the packed code buffer for an N x K matrix; 0 if the shape is invalid.  (Sizes of
 * this library's own packed layout: no passage of the pages defines them.) */
size_t w4_packed_bytes(int N, int K, int bits, int group);

/* Bytes of EACH of the packed scales and zeros buffers; 0 if the shape is invalid.  (Likewise
 * library-defined.) */
size_t w4_packed_sz_bytes(int N, int K, int group);

/* Repack one matrix from the canonical format (host memory in, host memory out).
 * codes_hi must be NULL for bits == 4 and non-NULL for bits == 5.  Output buffers must hold
 * w4_packed_bytes / w4_packed_sz_bytes bytes.  Pure permutation: bit-exact, deterministic. */
int w4_repack(const uint8_t* codes_lo, const uint8_t* codes_hi, const uint16_t* scales,
              const uint16_t* zeros, int N, int K, int bits, int group, void* w_out,
              uint16_t* scales_out, uint16_t* zeros_out);

/* Repack a gate/up pair (each N x K, canonical, host) into the interleaved pair layout used by
 * w4_linear_swiglu.  Outputs hold w4_packed_bytes(2N,...) and w4_packed_sz_bytes(2N,...). */
int w4_repack_pair(const uint8_t* gate_lo, const uint8_t* gate_hi, const uint16_t* gate_scales,
                   const uint16_t* gate_zeros, const uint8_t* up_lo, const uint8_t* up_hi,
                   const uint16_t* up_scales, const uint16_t* up_zeros, int N, int K, int bits,
                   int group, void* w_pair_out, uint16_t* scales_pair_out,
                   uint16_t* zeros_pair_out);

/* out[T][N] = fp16_rne(X . dequant(W)^T).  x: fp16 [T][K] row-major, device.  w, scales, zeros:
 * w4_repack output, device.  out: fp16 [T][N], device.  T == 0 is a successful no-op.
 * Any T >= 1 is accepted; rows of x beyond T-1 are never read and rows of out beyond T-1
 * are never written. */
int w4_linear(const uint16_t* x, const void* w, const uint16_t* scales, const uint16_t* zeros,
              int T, int N, int K, int bits, int group, uint16_t* out, void* stream);

/* out[T][N] = fp16_rne(silu(X . Wg^T) * (X . Wu^T)), silu(a) = a / (1 + exp(-a)), in fp32.
 * N is the width of EACH of gate and up; w_pair/scales_pair/zeros_pair are w4_repack_pair
 * output (2N packed rows).  The gate_up pair of the ninfer-3080 performance notes ("The token
 * tile, and why it was hiding"). */
int w4_linear_swiglu(const uint16_t* x, const void* w_pair, const uint16_t* scales_pair,
                     const uint16_t* zeros_pair, int T, int N, int K, int bits, int group,
                     uint16_t* out, void* stream);

/* out[T][N] = fp16_rne(X . dequant(W)^T + R) with the add in fp32 (the LinearAdd op of the
 * ninfer-3080 performance notes, "A8 prefill routes" table).  residual: fp16 [T][N].
 * out == residual (exactly) is allowed: each element is read before it is written, once. */
int w4_linear_add(const uint16_t* x, const void* w, const uint16_t* scales, const uint16_t* zeros,
                  const uint16_t* residual, int T, int N, int K, int bits, int group,
                  uint16_t* out, void* stream);

/* ---- bf16 activations.  The same three ops with x, out (and residual) in bf16; weights,
 * scales and zero-points are the packed fp16 format above.  Each token row t is first copied to
 * the workspace as fp16 X[t] * 2^-e_t, with the power of two e_t (also stored in the workspace)
 * chosen from the row's largest magnitude so that the copy is exact for every value down to
 * 2^-17 of that magnitude; the kernel then runs the fp16 path and its epilogue scales the fp32
 * sums by 2^e_t, applies SwiGLU or adds the bf16 residual in fp32, and rounds once to bf16.
 * The pages' kernels run their activations in bf16 (ninfer-3080 performance notes, "What
 * changed", "Permuted k order").  Two kernels are enqueued per call (the copy, then the route
 * the fp16 op would take at the same T).  workspace: caller-owned device memory of at least
 * w4_bf16_workspace_bytes(T, K) bytes, 16-byte aligned, overlapping no argument; its contents
 * are scratch between calls.  Validation and errors as the fp16 calls, plus W4_ERR_INVALID_ARG
 * for a missing or short workspace and W4_ERR_ALIAS for an overlapping one. */
size_t w4_bf16_workspace_bytes(int T, int K); /* 0 if the shape is invalid */

int w4_linear_bf16(const uint16_t* x, const void* w, const uint16_t* scales, const uint16_t* zeros,
                   int T, int N, int K, int bits, int group, uint16_t* out, void* workspace,
                   size_t workspace_bytes, void* stream);

int w4_linear_swiglu_bf16(const uint16_t* x, const void* w_pair, const uint16_t* scales_pair,
                          const uint16_t* zeros_pair, int T, int N, int K, int bits, int group,
                          uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

int w4_linear_add_bf16(const uint16_t* x, const void* w, const uint16_t* scales,
                       const uint16_t* zeros, const uint16_t* residual, int T, int N, int K,
                       int bits, int group, uint16_t* out, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ---- A8 prefill route (lossy): int8 activations with a scale per 64 columns, int8 matrix-core
 * steps, the int32 partial sum of each 64-column group rescaled into fp32 (ninfer-3080
 * performance notes, "A8 prefill routes": per-group activation quantisation, held to a
 * relative L2 error of 0.04 against an fp64 oracle).  Per token row t and 64-column group g:
 * s[t][g] = max |x| / 127 and q[t][k] = rint(x[t][k] / s[t][g]) clamped to [-127, 127], both in
 * fp32 (a group of zeros: s = 0, q = 0); the call returns fp16(sum_k s q W^T) with the same
 * epilogues as the fp16 ops.  Requirements beyond the fp16 ops: group == 64 (else
 * W4_ERR_UNSUPPORTED) and integer zero-points in [0, 127] (any other zero-point turns the outputs
 * of the 128-row block that holds it into NaN).
 * workspace: caller-owned device memory of at least w4_a8_workspace_bytes(T, K) bytes, 16-byte
 * aligned, overlapping no argument.  Its layout: int8 codes [T][K] at offset 0, each 8-column run
 * stored as columns 0 4 1 5 2 6 3 7; fp32 scales at offset ceil16(T * K), as
 * [ceil(K / 128)][T][2] (group g of token t at [g / 2][t][g % 2]).
 * x may be NULL in the three ops: the workspace then already holds this T x K activation, as
 * written by w4_quantize_a8 (matrices that read one activation quantise it once).  Each op
 * enqueues the quantisation (unless x is NULL) and one GEMM kernel. */
size_t w4_a8_workspace_bytes(int T, int K); /* 0 if the shape is invalid */
int w4_quantize_a8(const uint16_t* x, int T, int K, void* workspace, size_t workspace_bytes,
                   void* stream);
int w4_linear_a8(const uint16_t* x, const void* w, const uint16_t* scales, const uint16_t* zeros,
                 int T, int N, int K, int bits, int group, uint16_t* out, void* workspace,
                 size_t workspace_bytes, void* stream);
int w4_linear_swiglu_a8(const uint16_t* x, const void* w_pair, const uint16_t* scales_pair,
                        const uint16_t* zeros_pair, int T, int N, int K, int bits, int group,
                        uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);
int w4_linear_add_a8(const uint16_t* x, const void* w, const uint16_t* scales, const uint16_t* zeros,
                     const uint16_t* residual, int T, int N, int K, int bits, int group,
                     uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---- allocation-free bf16 linear, for callers that cannot allocate device memory (code being
 * captured into a HIP graph, serving loops that must not call hipMalloc, harnesses that forbid
 * it).  Same arguments, results and validation as w4_linear_bf16 without the workspace: the
 * workspace is a static device array inside the library, W4_SCRATCH_BYTES bytes per device,
 * held by every device the library runs on until the process ends.  Calls whose
 * w4_bf16_workspace_bytes(T, K) exceeds W4_SCRATCH_BYTES return W4_ERR_SCRATCH.  The first
 * call on a device locates that device's array (a host-side symbol lookup, no allocation),
 * so make it once outside graph capture.  Every call on one device shares its array: calls
 * that overlap on one device (concurrent streams or threads) race and must be serialised by
 * the caller.  Nothing in the array needs to start at zero (each call writes what it reads).
 * Calls no hipMalloc, hipFree or allocating library routine. */
#define W4_SCRATCH_BYTES (32u << 20)
int w4_linear_bf16_noalloc(const uint16_t* x, const void* w, const uint16_t* scales,
                           const uint16_t* zeros, int T, int N, int K, int bits, int group,
                           uint16_t* out, void* stream);

/* ---- grouped call: several matrices that share one activation (ninfer-3080 performance notes,
 * "What changed": two parents over one activation; the projections that read one activation
 * with 4-bit and 5-bit weights).  One matrix of the group, as w4_repack output: */
typedef struct {
  const void* w;            /* packed codes of N rows x K columns */
  const uint16_t* scales;   /* packed scales */
  const uint16_t* zeros;    /* packed zero-points */
  int N;                    /* rows (multiple of 16) */
  int bits;                 /* 4 or 5; the matrices of a group may differ */
  uint16_t* out;            /* fp16 [T][N], caller-owned, written (not read) */
} w4_parent;

#define W4_MAX_PARENTS 4

/* out_p[T][N_p] = fp16_rne(X . dequant(W_p)^T) for p < nparents (1 .. W4_MAX_PARENTS), all
 * reading x [T][K].  For T <= 64 and K <= 5120 one kernel launch covers every matrix (each
 * workgroup runs the code width of its matrix) with the streaming kernel of that width (the
 * routes mfma_stream_t16 / _t32 / _t64 for T <= 16 / 32 / 64: each output equals that route's
 * single-matrix result bit for bit, which for 5-bit matrices at T > 32 is not the route
 * w4_linear picks); otherwise the call launches the route w4_route_for picks for each matrix,
 * one after another on `stream`.  Validation as w4_linear
 * for every matrix, and no output may overlap another matrix's output, packed data or x
 * (W4_ERR_ALIAS).  parents: host array, read during the call only. */
int w4_linear_grouped(const uint16_t* x, const w4_parent* parents, int nparents, int T, int K,
                      int group, void* stream);

/* ---- per-verify-width graphs: launch-overhead removal for decode steps.  A decode round calls
 * the same projections at a few token widths (concurrency x (draft + 1)); at one stream the
 * gaps and ramp-up/drain between short kernels are a large part of the step (ninfer-3080
 * performance notes, "What is left at C1"; Kernarc, "One decode step, top to silicon": one graph
 * per verify width).  A set records, per width, every library call (or any other capturable
 * work) the caller enqueues on `stream` between w4_graph_set_begin and w4_graph_set_end, and
 * w4_graph_set_launch replays that width's instantiated graph in one launch.  The buffers the
 * recorded calls name must stay allocated at the same addresses while the graph is replayed;
 * their contents are read at replay time.  One capture at a time per set; a width is recorded
 * once (begin on a recorded width is W4_ERR_INVALID_ARG).  The set allocates host memory only.
 * stream must not be NULL (the null stream cannot be captured). */
typedef struct w4_graph_set w4_graph_set;
w4_graph_set* w4_graph_set_create(void);  /* NULL if out of host memory */
int w4_graph_set_begin(w4_graph_set* set, int width, void* stream);  /* starts stream capture */
int w4_graph_set_end(w4_graph_set* set, int width, void* stream);    /* ends it, instantiates */
int w4_graph_set_launch(w4_graph_set* set, int width, void* stream); /* W4_ERR_DOMAIN: not recorded */
int w4_graph_set_has(w4_graph_set* set, int width);                  /* 1 if recorded, else 0 */
void w4_graph_set_destroy(w4_graph_set* set);

/* ---- routes: every op has several kernels ("schedules"), each with an explicit T domain
 * (ninfer-3080 performance notes, "Route boundaries are measured here").  The three calls
 * above pick exactly one route with w4_route_for and launch it once. */

/* Route id chosen for (op, bits, T, N, K), or a negative w4_status. */
int w4_route_for(int op, int bits, int T, int N, int K);

/* Run a specific route; W4_ERR_DOMAIN if T lies outside its domain.  residual is ignored
 * unless op == W4_OP_ADD.  Same argument meaning and validation as the op's own call. */
int w4_linear_route(int route_id, int op, const uint16_t* x, const void* w,
                    const uint16_t* scales, const uint16_t* zeros, const uint16_t* residual,
                    int T, int N, int K, int bits, int group, uint16_t* out, void* stream);

/* Run a specific route with bf16 activations (as w4_linear_route, with the workspace of the
 * bf16 calls above). */
int w4_linear_route_bf16(int route_id, int op, const uint16_t* x, const void* w,
                         const uint16_t* scales, const uint16_t* zeros, const uint16_t* residual,
                         int T, int N, int K, int bits, int group, uint16_t* out, void* workspace,
                         size_t workspace_bytes, void* stream);

int w4_route_count(void);
const char* w4_route_name(int route_id); /* NULL for an unknown id */
/* T domain [*tmin, *tmax] of a route; W4_ERR_DOMAIN for an unknown id. */
int w4_route_domain(int route_id, int* tmin, int* tmax);

/* Library plumbing; no passage of the pages defines these two.  w4_status_str: a static,
 * NUL-terminated description of a w4_status (never NULL; "unknown status" for other values).
 * w4_layout_version: W4_LAYOUT_VERSION of the packed layout this library reads and writes. */
const char* w4_status_str(int status);
int w4_layout_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4GEMM_H */
