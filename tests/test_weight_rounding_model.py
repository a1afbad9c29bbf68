"""CPU model of the kernels' weight arithmetic on the SwiGLU pair with outlier channels.

Every kernel forms the dequantised weight in fp16, w16 = fp16_rne((q - z) * s) (q - z is exact
for integer zero-points, so this is one rounding per weight), multiplies it with the fp16
activations in the matrix cores and accumulates in fp32.  This test evaluates that arithmetic
in numpy (fp64 sums of x * w16, which is at least as accurate as the fp32 accumulation), on the
inputs of the GPU full-K test: N = 784 rows, activations N(0, 0.5^2) with 8 channels scaled x30
(the outlier channels of the ninfer-3080 performance notes, "cuBLAS prefill route").

It records the reading the library states about its tolerance: the relative L2 bound holds with
room to spare, but the per-element bound |y - y_ref| <= 1e-2 (1 + |y_ref|) does not hold for the
SwiGLU pair on every input, whatever the kernel: silu(gate) * up multiplies the up projection's
absolute rounding error by silu(gate) and the gate's by |up|, while y itself can stay small.  The
x30 channels make those factors large, and so does a long K with 5-bit codes (K = 17408 below).
The largest element error grows with K, with 5-bit codes, with outlier channels and with the
number of outputs, while the relative L2 error stays near 3.5e-4.  The configured SwiGLU workload
(4-bit, K = 5120, N(0, 0.5^2), no outlier channels) meets both bounds over all of its outputs at
every measured width (6.2e-3 at T = 64, the largest); the GPU tests hold 4-bit pairs to both
bounds at K <= 5120 without outlier channels, and 5-bit pairs (1.29e-2 with 4096 rows at
K = 5056) and longer K to the relative L2 bound.  Single matrices
(linear, LinearAdd) meet both bounds with outlier channels (GPU tests at full size and full K)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import make_activations, make_weights

N = 784


def _w16(ws, K, bits):
    q = oracle.unpack_codes(ws.lo, ws.hi, K, bits).astype(np.float64)
    z = np.repeat(ws.zeros.astype(np.float64), 64, axis=1)
    s = np.repeat(ws.scales.astype(np.float64), 64, axis=1)
    return ((q - z) * s).astype(np.float16).astype(np.float64)


def _case(K, bits, outliers):
    rng = np.random.default_rng(K + 10 * bits + 1)  # the GPU full-K test's seed for the pair
    scale = (0.0025, 0.01) if bits == 5 else (0.005, 0.02)
    g = make_weights(rng, "w", N, K, bits, ("uniform", 6, 9), scale)
    u = make_weights(rng, "u", N, K, bits, ("uniform", 6, 9), scale)
    x, _ = make_activations(rng, 64, K, 0.5, outliers)
    ref = oracle.swiglu(x, (g.lo, g.hi, g.scales, g.zeros), (u.lo, u.hi, u.scales, u.zeros), bits=bits)
    x64 = x.astype(np.float64)
    model = oracle.fp16_round(oracle.silu(x64 @ _w16(g, K, bits).T) * (x64 @ _w16(u, K, bits).T))
    model = model.astype(np.float64)
    rel = oracle.rel_l2(model, ref)
    elem = float(np.max(np.abs(model - ref) / (1.0 + np.abs(ref))))
    return rel, elem


@pytest.mark.parametrize("K,bits,elem_lo", [(5056, 4, 1.1e-2), (5120, 5, 2.5e-2), (5056, 5, 2.5e-2)])
def test_swiglu_outliers_exceed_element_bound(K, bits, elem_lo):
    """The fp16-weight arithmetic alone exceeds the element bound (recorded: 1.20e-2 at K = 5056
    with 4-bit codes, 2.9e-2 with 5-bit codes), while rel L2 stays near 3.3e-4."""
    rel, elem = _case(K, bits, 8)
    print(f"K={K} bits={bits}: rel_l2={rel:.3e} max_elem={elem:.3e}")
    assert rel <= 5e-4
    assert elem > elem_lo


@pytest.mark.parametrize("K,bits", [(5120, 4), (5056, 4), (5120, 5), (5056, 5)])
def test_swiglu_without_outliers_inside_both_bounds(K, bits):
    """The configured SwiGLU distribution (no outlier channels): both bounds hold."""
    rel, elem = _case(K, bits, 0)
    print(f"K={K} bits={bits}: rel_l2={rel:.3e} max_elem={elem:.3e}")
    assert rel <= 2e-3 and elem <= 1e-2


def _long_k_case(K, bits, T):
    """The GPU long-K test's SwiGLU case: N = 48, no outlier channels, its seed."""
    rng = np.random.default_rng(K + T + bits + 1)
    scale = (0.0025, 0.01) if bits == 5 else (0.005, 0.02)
    g = make_weights(rng, "w", 48, K, bits, ("uniform", 6, 9), scale)
    u = make_weights(rng, "u", 48, K, bits, ("uniform", 6, 9), scale)
    x, _ = make_activations(rng, T, K, 0.5, 0)
    ref = oracle.swiglu(x, (g.lo, g.hi, g.scales, g.zeros), (u.lo, u.hi, u.scales, u.zeros), bits=bits)
    x64 = x.astype(np.float64)
    model = oracle.fp16_round(oracle.silu(x64 @ _w16(g, K, bits).T) * (x64 @ _w16(u, K, bits).T))
    model = model.astype(np.float64)
    return oracle.rel_l2(model, ref), float(np.max(np.abs(model - ref) / (1.0 + np.abs(ref))))


def test_swiglu_long_k_5bit_exceeds_element_bound():
    """5-bit codes at K = 17408, T = 32, no outliers: 1.68e-2 (an output near 0.31 whose gate
    is 9.3: silu(gate) multiplies the up projection's rounding error)."""
    rel, elem = _long_k_case(17408, 5, 32)
    print(f"K=17408 bits=5 T=32: rel_l2={rel:.3e} max_elem={elem:.3e}")
    assert rel <= 5e-4 and elem > 1.5e-2


def test_swiglu_5bit_many_outputs_exceed_element_bound():
    """5-bit codes at K = 5056 without outlier channels, 4096 output rows, T = 32 (the K-split
    route's GPU test case, its seed): 1.29e-2, the GPU kernel's own figure to three digits."""
    N, K, T, bits = 4096, 5056, 32, 5
    rng = np.random.default_rng(N + K + T + 7 * bits + 31 * 1)
    scale = (0.0025, 0.01)
    g = make_weights(rng, "w", N, K, bits, ("uniform", 6, 9), scale)
    u = make_weights(rng, "u", N, K, bits, ("uniform", 6, 9), scale)
    x, _ = make_activations(rng, T, K, 0.5, 0)
    ref = oracle.swiglu(x, (g.lo, g.hi, g.scales, g.zeros), (u.lo, u.hi, u.scales, u.zeros), bits=bits)
    x64 = x.astype(np.float64)
    model = oracle.fp16_round(oracle.silu(x64 @ _w16(g, K, bits).T) * (x64 @ _w16(u, K, bits).T))
    model = model.astype(np.float64)
    rel = oracle.rel_l2(model, ref)
    elem = float(np.max(np.abs(model - ref) / (1.0 + np.abs(ref))))
    print(f"N={N} K={K} bits=5 T={T}: rel_l2={rel:.3e} max_elem={elem:.3e}")
    assert rel <= 5e-4 and elem > 1.2e-2


def test_swiglu_more_outputs_exceed_element_bound():
    """More outputs, larger extremes: 5-bit codes, K = 12352, T = 300 (the wide route's width in
    the GPU long-K test): 2.2e-2."""
    rel, elem = _long_k_case(12352, 5, 300)
    print(f"K=12352 bits=5 T=300: rel_l2={rel:.3e} max_elem={elem:.3e}")
    assert rel <= 5e-4 and elem > 2e-2


@pytest.mark.parametrize("K,bits", [(6144, 4), (12352, 4), (17408, 4), (6144, 5), (12352, 5), (17408, 5)])
def test_swiglu_long_k_relative_l2(K, bits):
    for T in (1, 3, 32, 65, 300):
        rel, _ = _long_k_case(K, bits, T)
        assert rel <= 1e-3, (K, bits, T, rel)
