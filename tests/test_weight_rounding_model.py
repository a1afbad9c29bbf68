"""CPU model of the kernels' weight arithmetic on the SwiGLU pair with outlier channels.

Every kernel forms the dequantised weight in fp16, w16 = fp16_rne((q - z) * s) (q - z is exact
for integer zero-points, so this is one rounding per weight), multiplies it with the fp16
activations in the matrix cores and accumulates in fp32.  This test evaluates that arithmetic
in numpy (fp64 sums of x * w16, which is at least as accurate as the fp32 accumulation), on the
inputs of the GPU full-K test: N = 784 rows, activations N(0, 0.5^2) with 8 channels scaled x30
(the outlier channels of the ninfer-3080 performance notes, "cuBLAS prefill route").

It records the reading the library states about its tolerance: the relative L2 bound holds with
room to spare, but the per-element bound |y - y_ref| <= 1e-2 (1 + |y_ref|) does not hold for the
SwiGLU pair on such inputs, whatever the kernel: silu(gate) * up multiplies the gate's absolute
rounding error by |up|, which the x30 channels make large, while a small gate keeps |y| small.
The configured SwiGLU workload (N(0, 0.5^2), no outlier channels) is inside the domain where
both bounds hold; single matrices (linear, LinearAdd) meet both bounds with outlier channels
(GPU tests at full size and full K)."""
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
