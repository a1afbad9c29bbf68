"""GPU tier: the register-ring kernels (routes mfma_reg_t16 / _t32 / _t64, mfma_reg32_t32 / _t64).

Each workgroup takes an even share of the row tiles (one workgroup per compute unit, up to six
16-row tiles, or five gate / up tile pairs for the SwiGLU op); the row counts below give every
instance size, shares that differ by one unit (the last unit of a share is then absent), and
grids of more than one round.  K covers waves without any k-block (K = 320: three blocks for
four waves), a half-size last block, ring loops with a remainder, and long rows.  Every output
is compared with the fp64 oracle.
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

# units (16-row tiles, or tile pairs for SwiGLU) -> largest share with 256 workgroups:
# 100 -> 1, 300 -> 2, 600 -> 3, 900 -> 4, 1200 -> 5, 1500 -> 6 (linear cap), 1700 -> 6 in
# 284 workgroups; SwiGLU: 1400 -> 5 pairs in 280 workgroups
LINEAR_UNITS = [100, 300, 600, 900, 1200, 1500, 1700]
SWIGLU_UNITS = [100, 300, 600, 900, 1200, 1400]
ROUTE_T = [("mfma_reg_t16", 1), ("mfma_reg_t16", 16), ("mfma_reg_t32", 17), ("mfma_reg_t32", 32),
           ("mfma_reg_t64", 33), ("mfma_reg_t64", 64), ("mfma_reg32_t32", 1), ("mfma_reg32_t32", 20),
           ("mfma_reg32_t32", 32), ("mfma_reg32_t64", 33), ("mfma_reg32_t64", 64)]


def route_id(name):
    return {w4.route_name(i): i for i in range(w4.route_count())}[name]


def _run(route, op, N, K, T, bits, seed, zero=("uniform", 6, 9)):
    rng = np.random.default_rng(seed)
    scale = (0.0025, 0.01) if bits == 5 else (0.005, 0.02)
    ws = [make_weights(rng, "w", N, K, bits, zero, scale)]
    if op == w4.OP_SWIGLU:
        ws.append(make_weights(rng, "u", N, K, bits, zero, scale))
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
    # the SwiGLU pair is held to the relative L2 bound only beyond K = 5120: its largest element
    # error grows with K (the fp16-weight arithmetic alone exceeds the element bound there:
    # tests/test_weight_rounding_model.py)
    assert_close(to_np(y), ref, f"{route} op{op} b{bits} T{T} N{N} K{K}",
                 elem=not (op == w4.OP_SWIGLU and K > 5120))


@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("units", LINEAR_UNITS)
@pytest.mark.parametrize("route,T", ROUTE_T)
def test_regring_linear_shares(route, T, units, bits):
    _run(route, w4.OP_LINEAR, 16 * units, 320, T, bits, seed=units + T + bits)


@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("units", SWIGLU_UNITS)
@pytest.mark.parametrize("route,T", ROUTE_T)
def test_regring_swiglu_shares(route, T, units, bits):
    _run(route, w4.OP_SWIGLU, 16 * units, 320, T, bits, seed=3 * units + T + bits)


# K = 1088: a half-size last block; 2112: 17 blocks over four waves (5, 4, 4, 4: ring loops
# with a remainder); 6208: 48 blocks and a half; 17408: 136 blocks
@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("K", [1088, 2112, 6208, 17408])
@pytest.mark.parametrize("route,T", [("mfma_reg_t16", 7), ("mfma_reg_t32", 20), ("mfma_reg_t64", 64),
                                     ("mfma_reg32_t32", 20), ("mfma_reg32_t32", 24), ("mfma_reg32_t64", 64)])
@pytest.mark.parametrize("op", [w4.OP_LINEAR, w4.OP_SWIGLU, w4.OP_ADD])
def test_regring_k_lengths(op, route, T, K, bits):
    _run(route, op, 16 * 40, K, T, bits, seed=K + T + op + bits)


# The 32-row form splits K over the workgroups of a pair group when K has at least 64 blocks
# and the split shortens the largest share; the slice count follows from the shape: 5120 rows
# at K = 8192 take three slices, 3200 rows two, 640 rows at K = 12352 four (with a half-size
# last block), the 640-row SwiGLU pair (40 pairs) four.
SPLIT_CASES = [(w4.OP_LINEAR, 5120, 8192), (w4.OP_ADD, 3200, 8192), (w4.OP_LINEAR, 640, 12352),
               (w4.OP_SWIGLU, 640, 12352)]


@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("route,T", [("mfma_reg32_t32", 1), ("mfma_reg32_t32", 32), ("mfma_reg32_t64", 64)])
@pytest.mark.parametrize("op,N,K", SPLIT_CASES)
def test_regring32_k_split(op, N, K, route, T, bits):
    _run(route, op, N, K, T, bits, seed=N + K + T + bits + op)


@pytest.mark.parametrize("route,T", [("mfma_reg_t16", 5), ("mfma_reg_t64", 40)])
def test_regring_fractional_zero_points(route, T):
    # zero-points with a fraction take the exact split into integer and fractional parts
    _run(route, w4.OP_LINEAR, 16 * 300, 1088, T, 4, seed=T, zero=("real", 3.0, 12.0))


@pytest.mark.parametrize("route,N,K", [("mfma_reg_t16", 16 * 900, 2048), ("mfma_reg_t32", 16 * 900, 2048),
                                       ("mfma_reg_t64", 16 * 900, 2048), ("mfma_reg32_t32", 16 * 900, 2048),
                                       ("mfma_reg32_t64", 640, 12352)])
def test_regring_deterministic(route, N, K):
    T, bits = 16, 4
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


# ---- the K split's workspace: static device slots, one per stream (four), so that split calls
# on different streams never share partial sums; a stream without a slot runs unsplit.
def _split_inputs(seed, N=640, K=12352, T=32, bits=4):
    rng = np.random.default_rng(seed)
    w = make_weights(rng, "w", N, K, bits, ("uniform", 6, 9), (0.005, 0.02))
    x, _ = make_activations(rng, T, K, 1.0, 0)
    ref = oracle.linear(x, *canon(w), bits=bits)
    return torch.from_numpy(x).to(DEV), w4.pack_weight(*canon(w), bits, device=DEV), ref


def test_regring32_split_on_overlapping_streams():
    rid = route_id("mfma_reg32_t32")
    cases = [_split_inputs(100 + i) for i in range(6)]
    streams = [torch.cuda.Stream() for _ in range(6)]
    torch.cuda.synchronize()
    outs = [[] for _ in range(6)]
    print("case split on 6 streams, 3 rounds", flush=True)
    for _ in range(3):
        for i, (s, (x, pw, _)) in enumerate(zip(streams, cases)):
            with torch.cuda.stream(s):
                outs[i].append(w4.linear_route(rid, w4.OP_LINEAR, x, pw))
    torch.cuda.synchronize()
    for i, (_, _, ref) in enumerate(cases):
        for y in outs[i]:
            assert_close(to_np(y), ref, f"stream {i}")
        assert all(torch.equal(y.view(torch.int16), outs[i][0].view(torch.int16)) for y in outs[i])


@pytest.mark.parametrize("op", [w4.OP_LINEAR, w4.OP_SWIGLU])
def test_regring32_split_graph_replays(op):
    N, K, T, bits = 640, 12352, 24, 5
    rng = np.random.default_rng(7 + op)
    ws = [make_weights(rng, "w", N, K, bits, ("const", 16), (0.0025, 0.01))]
    xn = make_activations(rng, T, K, 0.5 if op == w4.OP_SWIGLU else 1.0, 0)[0]
    if op == w4.OP_SWIGLU:
        ws.append(make_weights(rng, "u", N, K, bits, ("const", 16), (0.0025, 0.01)))
        pw = w4.pack_pair(canon(ws[0]), canon(ws[1]), bits, device=DEV)
        ref = oracle.swiglu(xn, canon(ws[0]), canon(ws[1]), bits=bits)
    else:
        pw = w4.pack_weight(*canon(ws[0]), bits, device=DEV)
        ref = oracle.linear(xn, *canon(ws[0]), bits=bits)
    x = torch.from_numpy(xn).to(DEV)
    rid = route_id("mfma_reg32_t32")
    print(f"case split graph op={op}", flush=True)
    eager = w4.linear_route(rid, op, x, pw)
    torch.cuda.synchronize()
    static_out = torch.empty((T, N), dtype=torch.float16, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w4.linear_route(rid, op, x, pw, out=static_out)
    first = None
    for rep in range(4):
        static_out.fill_(float("nan"))
        again = w4.linear_route(rid, op, x, pw)  # eager split calls of the program between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), eager.view(torch.int16))
        assert_close(to_np(static_out), ref, f"replay {rep}", elem=op != w4.OP_SWIGLU)
        if first is None:
            first = static_out.clone()
        assert torch.equal(static_out.view(torch.int16), first.view(torch.int16))


# An odd number of 16-row tiles leaves the 32-row form's last pair without its second tile (its
# lanes re-read the first tile, whose rows there are never stored): unsplit (K = 2112) and with
# the K split (K = 12352, 41 tiles: 21 pairs in four slices).
@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("op", [w4.OP_LINEAR, w4.OP_ADD])
@pytest.mark.parametrize("route,T", [("mfma_reg32_t32", 9), ("mfma_reg32_t64", 40)])
@pytest.mark.parametrize("tiles,K", [(301, 2112), (41, 12352), (1, 640)])
def test_regring32_odd_tile_count(tiles, K, route, T, op, bits):
    _run(route, op, 16 * tiles, K, T, bits, seed=tiles + K + T + op + bits)
