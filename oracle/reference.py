"""fp64 oracle: dequantise the canonical codes, then multiply.  Test infrastructure only.

Sources (the pages this library is built from):

* ninfer-3080 performance notes, section "cuBLAS prefill route" (the result
  paragraph and the quality-trade paragraph that follows it): the integer route
  keeps one scale per 64 columns of the weight; a per-channel factor folded out
  of the activations and into the weights leaves the product unchanged.
* ninfer-3080 performance notes, section "What changed" (bullets "Permuted k
  order" and the Q5 small-T kernel): 4-bit codes; the 5-bit form is a 4-bit
  plane plus a high-bit plane; the k order inside a group is free.
* ninfer-3080 performance notes, section "A8 prefill routes" (route table):
  LinearAdd, a projection whose result is added to a residual.
* ARK research, "Fused kernels", section "Why standard kernels stall": a fused
  low-bit kernel returns the ordinary product of the activations with the
  dequantised weights; this oracle forms that product in two separate steps
  (dequantise everything, then multiply).

Readings where the pages are silent (each is listed with its reason in the
design notes): the dequantised weight is ``w = s * (q - z)`` with the zero-point
``z`` in code units; activations, scales, zero-points and the output are fp16;
SwiGLU is ``silu(gate) * up`` with ``silu(a) = a / (1 + exp(-a))``.

Everything is computed in float64 from exact fp16 -> fp64 conversions.  The
result is returned unrounded; ``fp16_round`` gives the round-to-nearest-even
fp16 value when a test needs it.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

GROUP = 64


def unpack_codes(lo: np.ndarray, hi: Optional[np.ndarray], K: int, bits: int) -> np.ndarray:
    """Codes q[n, k] as int64 from the canonical byte planes.

    4-bit: byte ``lo[n][k//2]`` holds code k in its low nibble when k is even and
    in its high nibble when k is odd.  5-bit: bit 4 comes from the high-bit
    plane, bit ``k % 8`` of ``hi[n][k//8]`` (ninfer-3080 performance notes,
    "What changed": the Q5 form is a 4-bit plane plus a high-bit plane).
    """
    lo = np.asarray(lo, dtype=np.uint8)
    N = lo.shape[0]
    if lo.shape != (N, K // 2):
        raise ValueError("lo must be [N, K/2]")
    q = np.empty((N, K), dtype=np.int64)
    q[:, 0::2] = lo & 0x0F
    q[:, 1::2] = lo >> 4
    if bits == 4:
        return q
    if bits != 5:
        raise ValueError("bits must be 4 or 5")
    hi = np.asarray(hi, dtype=np.uint8)
    if hi.shape != (N, K // 8):
        raise ValueError("hi must be [N, K/8]")
    for i in range(8):
        q[:, i::8] += ((hi >> i) & 1).astype(np.int64) << 4
    return q


def dequantize(q: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
               group: int = GROUP) -> np.ndarray:
    """W[n, k] = s[n, k // group] * (q[n, k] - z[n, k // group]) in fp64.

    One scale and one zero-point per ``group`` consecutive K-columns (64 on the
    pages: ninfer-3080 performance notes, "cuBLAS prefill route").
    """
    N, K = q.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    s = np.asarray(scales).astype(np.float64)
    z = np.asarray(zeros).astype(np.float64)
    if s.shape != (N, K // group) or z.shape != (N, K // group):
        raise ValueError("scales/zeros must be [N, K/group]")
    s_full = np.repeat(s, group, axis=1)
    z_full = np.repeat(z, group, axis=1)
    return s_full * (q.astype(np.float64) - z_full)


def linear(x: np.ndarray, lo: np.ndarray, hi: Optional[np.ndarray], scales: np.ndarray,
           zeros: np.ndarray, bits: int, group: int = GROUP,
           n_chunk: int = 2048) -> np.ndarray:
    """Y[t, n] = sum_k X[t, k] * W[n, k], i.e. Y = X . dequant(Wq)^T, in fp64.

    The N dimension is processed in chunks only to bound host memory; each
    output element is one plain fp64 dot product over all of K.
    """
    x64 = np.asarray(x).astype(np.float64)
    T, K = x64.shape
    N = lo.shape[0]
    y = np.empty((T, N), dtype=np.float64)
    for n0 in range(0, N, n_chunk):
        n1 = min(N, n0 + n_chunk)
        q = unpack_codes(lo[n0:n1], None if hi is None else hi[n0:n1], K, bits)
        w = dequantize(q, scales[n0:n1], zeros[n0:n1], group)
        y[:, n0:n1] = x64 @ w.T
    return y


def linear_rows(x: np.ndarray, lo: np.ndarray, hi: Optional[np.ndarray], scales: np.ndarray,
                zeros: np.ndarray, bits: int, rows: Sequence[int],
                group: int = GROUP) -> np.ndarray:
    """Y[:, rows] only (for sampled checks at full size): fp64, shape [T, len(rows)]."""
    rows = np.asarray(rows, dtype=np.int64)
    K = np.asarray(x).shape[1]
    q = unpack_codes(lo[rows], None if hi is None else hi[rows], K, bits)
    w = dequantize(q, scales[rows], zeros[rows], group)
    return np.asarray(x).astype(np.float64) @ w.T


def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a / (1 + exp(-a)), written to stay finite for large |a|."""
    a = np.asarray(a, dtype=np.float64)
    out = np.empty_like(a)
    pos = a >= 0
    out[pos] = a[pos] / (1.0 + np.exp(-a[pos]))
    e = np.exp(a[~pos])
    out[~pos] = a[~pos] * e / (1.0 + e)
    return out


def swiglu(x, gate, up, bits: int, group: int = GROUP) -> np.ndarray:
    """out = silu(X . Wg^T) * (X . Wu^T) in fp64.

    ``gate`` and ``up`` are (lo, hi, scales, zeros) tuples in canonical form.
    The gate/up pair is the MLP's gate_up projection (ninfer-3080 performance
    notes, "The token tile, and why it was hiding": gate_up pairing).
    """
    g = linear(x, *gate, bits=bits, group=group)
    u = linear(x, *up, bits=bits, group=group)
    return silu(g) * u


def linear_add(x, lo, hi, scales, zeros, r, bits: int, group: int = GROUP) -> np.ndarray:
    """out = X . W^T + R in fp64 (the LinearAdd op of the ninfer-3080 notes, A8 routes table)."""
    return linear(x, lo, hi, scales, zeros, bits, group) + np.asarray(r).astype(np.float64)


A8_GROUP = 64


def quantize_a8(x: np.ndarray, group: int = A8_GROUP):
    """Per-(token, group) symmetric int8 activations of the A8 prefill route.

    The ninfer-3080 performance notes ("A8 prefill routes", and the quality paragraph of
    "cuBLAS prefill route") quantise the activations to int8 with a scale per 64 columns and
    hold the result to a relative L2 error of 0.04 against an fp64 oracle; they give no formula.
    Reading: per token row and 64-column group, m = max |x|, scale s = m / 127 and code
    q = rint(x / s) (round half to even) clamped to [-127, 127], both divisions in fp32; a
    group of zeros has s = 0 and q = 0.  Returns (q int8 [T, K], s float32 [T, K / group])."""
    x32 = np.asarray(x).astype(np.float32)
    T, K = x32.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    xg = x32.reshape(T, K // group, group)
    m = np.max(np.abs(xg), axis=2)
    s = (m / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint(xg / safe[:, :, None])
    q = np.where(s[:, :, None] > 0, q, 0.0)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q.reshape(T, K), s


def linear_a8(x, lo, hi, scales, zeros, bits: int, group: int = GROUP) -> np.ndarray:
    """The A8 route's product in fp64: Y = Xa . dequant(W)^T with Xa[t, k] = s[t, g] * q[t, k]
    the int8 activations of quantize_a8 (groups of 64 columns)."""
    q, s = quantize_a8(x)
    xa = q.astype(np.float64) * np.repeat(s.astype(np.float64), A8_GROUP, axis=1)
    return linear(xa, lo, hi, scales, zeros, bits, group)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> their exact values in fp64.

    A bfloat16 number is the upper 16 bits of an IEEE binary32 number (sign, 8 exponent bits,
    7 mantissa bits), so its value is that of the binary32 word ``bits << 16``.  Used for the
    bf16-activation calls, whose inputs and outputs are bf16 (the pages' kernels run their
    activations in bf16: ninfer-3080 performance notes, "What changed")."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp16_round(y: np.ndarray) -> np.ndarray:
    """Round fp64 values to fp16 with round-to-nearest-even (numpy's cast)."""
    return np.asarray(y, dtype=np.float64).astype(np.float16)


def rel_l2(y: np.ndarray, ref: np.ndarray) -> float:
    """||y - ref||_2 / ||ref||_2 in fp64 (0 if both are zero)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((y - ref).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
