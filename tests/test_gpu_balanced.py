"""GPU tier: the balanced partition of the warp-specialised kernel (routes mfma_bal_t32 / _t64).

Each workgroup takes an even share of the row tiles (one workgroup per compute unit, up to five
32-row pairs each); the row counts below give every instance size, 1 to 5 pairs per workgroup,
shares that start on odd tiles and end in a half-empty pair, and a grid of more than one round.
Every output is compared with the fp64 oracle.
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

# output columns N -> tiles of 16 rows (linear) or pairs of gate/up tiles (SwiGLU); with 256
# workgroups the largest share is ceil(units / 256): tiles 2 / 4 / 6 / 8 / 10 / 10 in 261
# workgroups (linear), pairs 1 / 2 / 3 / 4 / 5 / 5 in 261 workgroups (SwiGLU)
LINEAR_N = [16 * 300, 16 * 700, 16 * 1100, 16 * 1800, 16 * 2200, 16 * 2600]
SWIGLU_N = [16 * 200, 16 * 500, 16 * 700, 16 * 1000, 16 * 1100, 16 * 1300]


def route_id(name):
    return {w4.route_name(i): i for i in range(w4.route_count())}[name]


def _run(route, op, N, K, T, bits, seed):
    rng = np.random.default_rng(seed)
    scale = (0.0025, 0.01) if bits == 5 else (0.005, 0.02)
    ws = [make_weights(rng, "w", N, K, bits, ("uniform", 6, 9), scale)]
    if op == w4.OP_SWIGLU:
        ws.append(make_weights(rng, "u", N, K, bits, ("uniform", 6, 9), scale))
    x, _ = make_activations(rng, T, K, 0.5 if op == w4.OP_SWIGLU else 1.0, 0)
    r = make_residual(rng, T, N) if op == w4.OP_ADD else None
    if op == w4.OP_SWIGLU:
        pw = w4.pack_pair(canon(ws[0]), canon(ws[1]), bits, device=DEV)
        ref = oracle.swiglu(x, canon(ws[0]), canon(ws[1]), bits=bits)
    elif op == w4.OP_ADD:
        pw = w4.pack_weight(*canon(ws[0]), bits, device=DEV)
        ref = oracle.linear_add(x, *canon(ws[0]), r, bits=bits)
    else:
        pw = w4.pack_weight(*canon(ws[0]), bits, device=DEV)
        ref = oracle.linear(x, *canon(ws[0]), bits=bits)
    print(f"case route={route} op={op} bits={bits} T={T} N={N} K={K}", flush=True)
    rd = torch.from_numpy(r).to(DEV) if r is not None else None
    y = w4.linear_route(route_id(route), op, torch.from_numpy(x).to(DEV), pw, residual=rd)
    torch.cuda.synchronize()
    assert_close(to_np(y), ref, f"{route} op{op} b{bits} T{T} N{N} K{K}")


@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("N", LINEAR_N)
@pytest.mark.parametrize("route,T", [("mfma_bal_t32", 1), ("mfma_bal_t32", 32),
                                     ("mfma_bal_t64", 33), ("mfma_bal_t64", 64)])
def test_balanced_linear_shares(route, T, N, bits):
    _run(route, w4.OP_LINEAR, N, 320, T, bits, seed=N + T + bits)


@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("N", SWIGLU_N)
@pytest.mark.parametrize("route,T", [("mfma_bal_t32", 5), ("mfma_bal_t32", 32),
                                     ("mfma_bal_t64", 40), ("mfma_bal_t64", 64)])
def test_balanced_swiglu_shares(route, T, N, bits):
    _run(route, w4.OP_SWIGLU, N, 320, T, bits, seed=3 * N + T + bits)


@pytest.mark.parametrize("N", [16 * 700, 16 * 2200])
@pytest.mark.parametrize("T", [7, 64])
def test_balanced_add_long_k(N, T):
    route = "mfma_bal_t64" if T > 32 else "mfma_bal_t32"
    _run(route, w4.OP_ADD, N, 1088, T, 4, seed=N + 5 * T)


@pytest.mark.parametrize("route", ["mfma_bal_t32", "mfma_bal_t64"])
def test_balanced_deterministic(route):
    N, K, T, bits = 16 * 1100, 512, 32, 4
    rng = np.random.default_rng(11)
    ws = make_weights(rng, "w", N, K, bits, ("uniform", 6, 9), (0.005, 0.02))
    x, _ = make_activations(rng, T, K, 1.0, 0)
    pw = w4.pack_weight(*canon(ws), bits, device=DEV)
    xd = torch.from_numpy(x).to(DEV)
    rid = route_id(route)
    first = to_np(w4.linear_route(rid, w4.OP_LINEAR, xd, pw)).view(np.uint16)
    for _ in range(4):
        again = to_np(w4.linear_route(rid, w4.OP_LINEAR, xd, pw)).view(np.uint16)
        assert np.array_equal(first, again)
