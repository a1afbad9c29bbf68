"""Seeded synthetic workloads in the canonical groupwise weight format.

Canonical (user-side) format, the one both the oracle and the repacker read:

* 4-bit codes: ``lo`` is uint8 ``[N][K/2]``; code (n, k) is
  ``(lo[n][k//2] >> (4*(k & 1))) & 0xF`` -- the even k sits in the low nibble.
* 5-bit codes: the same 4-bit ``lo`` plane holds bits 0..3, and ``hi`` is uint8
  ``[N][K/8]`` holding bit 4: ``(hi[n][k//8] >> (k & 7)) & 1``.  This follows the
  split into a 4-bit plane plus a high-bit plane that the ninfer-3080
  performance notes describe for their Q5 kernels ("What changed", the Q5
  small-T bullet).
* ``scales`` and ``zeros``: float16 ``[N][K/64]``, one pair per 64 K-columns
  (ninfer-3080 performance notes, "cuBLAS prefill route": the integer route
  carries a scale per 64 columns).

Workload shapes are the projection shapes the ninfer-3080 performance notes
time ("What changed" table: 27B gate_up, attention input, GDN input; the A8
prefill routes table: Q5 [5120, 6144] LinearAdd).  Distributions follow the
configuration list this library is measured on; every draw is seeded.

Draw order per workload (fixed, so a seed names the bytes exactly): for each
weight matrix in order -- codes, zeros, scales; then X at the largest T, the
outlier channel indices, the x30 outlier factor in float32, rounding to fp16;
then the residual R.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

GROUP = 64


@dataclasses.dataclass
class WeightSet:
    name: str
    N: int
    K: int
    bits: int
    q: np.ndarray          # uint8 [N, K] raw codes (convenience for tests)
    lo: np.ndarray         # uint8 [N, K/2]
    hi: Optional[np.ndarray]  # uint8 [N, K/8] for 5-bit, else None
    scales: np.ndarray     # float16 [N, K/64]
    zeros: np.ndarray      # float16 [N, K/64]


@dataclasses.dataclass
class Workload:
    name: str
    weights: List[WeightSet]
    x: np.ndarray                  # float16 [Tmax, K]
    r: Optional[np.ndarray]        # float16 [Tmax, N] or None
    Ts: Tuple[int, ...]
    op: str                        # "linear" | "swiglu" | "add"
    outlier_idx: Optional[np.ndarray] = None


# name -> description.  "zero": ("const", z) or ("uniform", lo, hi) inclusive.
CONFIGS: Dict[str, dict] = {
    "tiny": dict(
        mats=[("w", 256, 512)], bits=4, zero=("const", 8), scale=(0.005, 0.02),
        x_sigma=1.0, outliers=0, Ts=(1,), op="linear"),
    "decode": dict(
        mats=[("w", 12288, 5120)], bits=4, zero=("uniform", 6, 9), scale=(0.005, 0.02),
        x_sigma=1.0, outliers=0, Ts=(1, 2, 4), op="linear"),
    "batched": dict(
        mats=[("attn_in", 7168, 5120), ("gdn_in", 4096, 5120)], bits=4,
        zero=("uniform", 6, 9), scale=(0.005, 0.02),
        x_sigma=1.0, outliers=8, Ts=(8, 16, 32, 64), op="linear"),
    "swiglu": dict(
        mats=[("gate", 17408, 5120), ("up", 17408, 5120)], bits=4,
        zero=("uniform", 6, 9), scale=(0.005, 0.02),
        x_sigma=0.5, outliers=0, Ts=(1, 4, 16, 64), op="swiglu"),
    "prefill": dict(
        mats=[("w", 5120, 6144)], bits=5, zero=("const", 16), scale=(0.0025, 0.01),
        x_sigma=1.0, outliers=8, Ts=(1024, 4096), op="add"),
    # shapes for route-boundary sweeps (not measured configurations): the 5-bit input projection
    # rows at K = 5120, the 5-bit down projection [5120, 17408], and 5120-row matrices at
    # K = 8192, 12288 (5-bit) and 8192, 17408 (4-bit) between the two
    "q5_k5120": dict(
        mats=[("w", 12288, 5120)], bits=5, zero=("const", 16), scale=(0.0025, 0.01),
        x_sigma=1.0, outliers=8, Ts=(1, 64), op="linear"),
    "q5_down": dict(
        mats=[("w", 5120, 17408)], bits=5, zero=("const", 16), scale=(0.0025, 0.01),
        x_sigma=1.0, outliers=8, Ts=(1, 64), op="linear"),
    "q5_k8192": dict(
        mats=[("w", 5120, 8192)], bits=5, zero=("const", 16), scale=(0.0025, 0.01),
        x_sigma=1.0, outliers=8, Ts=(1, 64), op="linear"),
    "q5_k12288": dict(
        mats=[("w", 5120, 12288)], bits=5, zero=("const", 16), scale=(0.0025, 0.01),
        x_sigma=1.0, outliers=8, Ts=(1, 64), op="linear"),
    "q4_k8192": dict(
        mats=[("w", 5120, 8192)], bits=4, zero=("uniform", 6, 9), scale=(0.005, 0.02),
        x_sigma=1.0, outliers=8, Ts=(1, 64), op="linear"),
    "q4_k17408": dict(
        mats=[("w", 5120, 17408)], bits=4, zero=("uniform", 6, 9), scale=(0.005, 0.02),
        x_sigma=1.0, outliers=8, Ts=(1, 64), op="linear"),
    # SwiGLU pairs smaller than the measured one: a 4096-row 4-bit pair and an 8192-row 5-bit
    # pair at K = 5120 (route-boundary sweeps only)
    "swiglu_4096": dict(
        mats=[("gate", 4096, 5120), ("up", 4096, 5120)], bits=4,
        zero=("uniform", 6, 9), scale=(0.005, 0.02),
        x_sigma=0.5, outliers=0, Ts=(1, 64), op="swiglu"),
    "swiglu_q5_8192": dict(
        mats=[("gate", 8192, 5120), ("up", 8192, 5120)], bits=5,
        zero=("const", 16), scale=(0.0025, 0.01),
        x_sigma=0.5, outliers=0, Ts=(1, 64), op="swiglu"),
}

OUTLIER_FACTOR = 30.0


def pack_canonical(q: np.ndarray, bits: int) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Write raw codes ``q`` (uint8 [N, K]) in the canonical byte format."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    low4 = q & 0xF
    lo = (low4[:, 0::2] | (low4[:, 1::2] << 4)).astype(np.uint8)
    if bits == 4:
        if q.max(initial=0) > 15:
            raise ValueError("4-bit codes must be < 16")
        return lo, None
    if bits != 5:
        raise ValueError("bits must be 4 or 5")
    if q.max(initial=0) > 31:
        raise ValueError("5-bit codes must be < 32")
    b4 = ((q >> 4) & 1).astype(np.uint8).reshape(N, K // 8, 8)
    hi = np.zeros((N, K // 8), dtype=np.uint8)
    for i in range(8):
        hi |= (b4[:, :, i] << i).astype(np.uint8)
    return lo, hi


def make_weights(rng: np.random.Generator, name: str, N: int, K: int, bits: int,
                 zero: Sequence, scale: Tuple[float, float], group: int = GROUP) -> WeightSet:
    """Draw codes, then zeros, then scales (in that order) for one matrix; one scale and one
    zero-point per `group` columns (64 in every measured configuration)."""
    if K % max(group, 64):
        raise ValueError("K must be a multiple of 64 (of 128 for groups of 128)")
    G = K // group
    q = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    if zero[0] == "const":
        zeros = np.full((N, G), zero[1], dtype=np.float16)
    elif zero[0] == "uniform":
        zeros = rng.integers(zero[1], zero[2] + 1, size=(N, G)).astype(np.float16)
    elif zero[0] == "real":  # continuous zero-points in [lo, hi), for fractional-z tests
        zeros = rng.uniform(zero[1], zero[2], size=(N, G)).astype(np.float16)
    else:
        raise ValueError(f"unknown zero spec {zero!r}")
    scales = rng.uniform(scale[0], scale[1], size=(N, G)).astype(np.float16)
    lo, hi = pack_canonical(q, bits)
    return WeightSet(name, N, K, bits, q, lo, hi, scales, zeros)


def make_activations(rng: np.random.Generator, T: int, K: int, sigma: float,
                     n_outliers: int, factor: float = OUTLIER_FACTOR
                     ) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """X ~ N(0, sigma^2) in fp16, with ``n_outliers`` channels scaled by ``factor``.

    The same channels are scaled for every token: outliers concentrate in a few
    input channels (ninfer-3080 performance notes, "cuBLAS prefill route").
    The factor is applied in float32 before the single rounding to fp16.
    """
    x = (rng.standard_normal((T, K)) * sigma).astype(np.float32)
    idx = None
    if n_outliers:
        idx = np.sort(rng.choice(K, n_outliers, replace=False))
        x[:, idx] *= np.float32(factor)
    return x.astype(np.float16), idx


def make_residual(rng: np.random.Generator, T: int, N: int) -> np.ndarray:
    return rng.standard_normal((T, N)).astype(np.float16)


def bf16_bits(x) -> np.ndarray:
    """float32 values -> bfloat16 bit patterns (uint16), rounded to nearest even: the input
    format of the bf16 calls (numpy has no bfloat16 type).  Finite inputs only."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def make_activations_bf16(rng: np.random.Generator, T: int, K: int, sigma: float,
                          n_outliers: int, factor: float = OUTLIER_FACTOR
                          ) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """As make_activations, rounded to bf16 instead of fp16: uint16 bit patterns [T, K]."""
    x = (rng.standard_normal((T, K)) * sigma).astype(np.float32)
    idx = None
    if n_outliers:
        idx = np.sort(rng.choice(K, n_outliers, replace=False))
        x[:, idx] *= np.float32(factor)
    return bf16_bits(x), idx


def make_workload(name: str, seed: int = 0, Ts: Optional[Sequence[int]] = None) -> Workload:
    """Build the named workload from ``CONFIGS`` with ``default_rng(seed)``."""
    cfg = CONFIGS[name]
    rng = np.random.default_rng(seed)
    ws = [make_weights(rng, nm, N, K, cfg["bits"], cfg["zero"], cfg["scale"])
          for (nm, N, K) in cfg["mats"]]
    K = cfg["mats"][0][2]
    Ts = tuple(Ts) if Ts is not None else tuple(cfg["Ts"])
    x, idx = make_activations(rng, max(Ts), K, cfg["x_sigma"], cfg["outliers"])
    r = None
    if cfg["op"] == "add":
        r = make_residual(rng, max(Ts), ws[0].N)
    return Workload(name, ws, x, r, Ts, cfg["op"], idx)
