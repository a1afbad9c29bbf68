"""GPU tier: degenerate shapes and closed forms on every route.

* the smallest legal shapes: one 16-row tile (the second tile of a 32-row pair is empty), one
  half-empty k-block (K = 64), one token;
* X = 0 gives Y = 0 and LinearAdd returns R bitwise; codes equal to their zero-point give 0;
* a single nonzero activation column reproduces the dequantised weight column exactly (checked
  at a ragged shape here; the one-hot test of test_gpu_parity.py covers every k).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w4_groupwise_gemm_amd as w4
from synth import make_weights, make_activations, make_residual
from gpu_util import assert_close, canon, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def routes():
    return [(w4.route_name(i), i) for i in range(w4.route_count())]


def _t_in(rid, T):
    lo, hi = w4.route_domain(rid)
    return max(lo, min(hi, T))


@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("N,K", [(16, 64), (16, 128), (48, 192), (32, 64)])
def test_smallest_shapes_every_route(N, K, bits):
    rng = np.random.default_rng(N * 7 + K + bits)
    scale = (0.0025, 0.01) if bits == 5 else (0.005, 0.02)
    for name, rid in routes():
        for op in (w4.OP_LINEAR, w4.OP_SWIGLU, w4.OP_ADD):
            for T0 in (1, 3, 17, 40, 70):
                T = _t_in(rid, T0)
                ws = [make_weights(rng, "w", N, K, bits, ("uniform", 6, 9), scale)]
                if op == w4.OP_SWIGLU:
                    ws.append(make_weights(rng, "u", N, K, bits, ("uniform", 6, 9), scale))
                    pw = w4.pack_pair(canon(ws[0]), canon(ws[1]), bits, device=DEV)
                else:
                    pw = w4.pack_weight(*canon(ws[0]), bits, device=DEV)
                x, _ = make_activations(rng, T, K, 1.0, 1)
                r = make_residual(rng, T, N)
                print(f"case edge route={name} op={op} bits={bits} T={T} N={N} K={K}", flush=True)
                y = w4.linear_route(rid, op, torch.from_numpy(x).to(DEV), pw,
                                    residual=torch.from_numpy(r).to(DEV) if op == w4.OP_ADD else None)
                if op == w4.OP_SWIGLU:
                    ref = oracle.swiglu(x, canon(ws[0]), canon(ws[1]), bits=bits)
                elif op == w4.OP_ADD:
                    ref = oracle.linear_add(x, *canon(ws[0]), r, bits=bits)
                else:
                    ref = oracle.linear(x, *canon(ws[0]), bits=bits)
                assert_close(to_np(y), ref, f"{name} op{op} b{bits} T{T} N{N} K{K}")


@pytest.mark.parametrize("bits", [4, 5])
def test_zero_activations(bits):
    """X = 0: Y = 0 exactly, and LinearAdd returns R bit for bit, on every route."""
    N, K = 96, 320
    rng = np.random.default_rng(41 + bits)
    ws = make_weights(rng, "w", N, K, bits, ("uniform", 6, 9), (0.005, 0.02))
    pw = w4.pack_weight(*canon(ws), bits, device=DEV)
    for name, rid in routes():
        T = _t_in(rid, 24)
        x = torch.zeros((T, K), dtype=torch.float16, device=DEV)
        r = torch.from_numpy(make_residual(rng, T, N)).to(DEV)
        y = w4.linear_route(rid, w4.OP_LINEAR, x, pw)
        assert torch.count_nonzero(y).item() == 0, name
        out = w4.linear_route(rid, w4.OP_ADD, x, pw, residual=r)
        assert torch.equal(out.view(torch.int16), r.view(torch.int16)), name


@pytest.mark.parametrize("bits", [4, 5])
def test_codes_at_zero_point_give_zero(bits):
    """q == z everywhere (integer z per group): every weight is 0, so Y = 0 exactly."""
    N, K = 64, 256
    rng = np.random.default_rng(53 + bits)
    ws = make_weights(rng, "w", N, K, bits, ("const", 0), (0.005, 0.02))
    G = K // 64
    zq = rng.integers(0, 1 << bits, size=(N, G))
    q = np.repeat(zq, 64, axis=1).astype(np.uint8)
    from synth.inputs import pack_canonical
    lo, hi = pack_canonical(q, bits)
    pw = w4.pack_weight(lo, hi, ws.scales, zq.astype(np.float16), bits, device=DEV)
    x, _ = make_activations(rng, 64, K, 1.0, 2)
    for name, rid in routes():
        T = _t_in(rid, 9)
        y = w4.linear_route(rid, w4.OP_LINEAR, torch.from_numpy(x[:T]).to(DEV), pw)
        assert torch.count_nonzero(y).item() == 0, name
