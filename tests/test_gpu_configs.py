"""GPU tier: every measured configuration at its full size, through the public calls the bench
times, checked against the fp64 oracle on sampled output columns (the oracle computes those
columns one by one over the full K).  One workload is built per configuration and reused for
all of its widths."""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import w4_groupwise_gemm_amd as w4
from synth import make_workload
from gpu_util import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NCOLS = 96  # sampled output columns per (configuration, width)

CASES = [("tiny", 1)] + [("decode", t) for t in (1, 2, 4)] + \
        [("batched", t) for t in (5, 8, 16, 20, 32, 64)] + [("swiglu", t) for t in (1, 4, 8, 16, 24, 64)] + \
        [("prefill", t) for t in (32, 128, 384, 1024, 4096)]
# batched 5, swiglu 8: the 8-row activation slice of the stream kernel at full K; batched 20,
# swiglu 24: its 32-row activation ring at full K; prefill 32: the 32-token route at K > 5120
# (narrow kernel); prefill 128, 384: the token-tiled narrow route


@functools.lru_cache(maxsize=1)
def _prepared(name):
    """(workload, packed device weight, canonical tuple or pair, op) for one configuration."""
    wl = make_workload(name)
    bits = wl.weights[0].bits
    if wl.op == "swiglu":
        g, u = wl.weights
        canon = ((g.lo, g.hi, g.scales, g.zeros), (u.lo, u.hi, u.scales, u.zeros))
        pw = w4.pack_pair(*canon, bits, device=DEV)
    else:
        # parents that share one activation run as one N-concatenated matrix
        lo = np.concatenate([ws.lo for ws in wl.weights])
        hi = None if bits == 4 else np.concatenate([ws.hi for ws in wl.weights])
        sc = np.concatenate([ws.scales for ws in wl.weights])
        ze = np.concatenate([ws.zeros for ws in wl.weights])
        canon = (lo, hi, sc, ze)
        pw = w4.pack_weight(*canon, bits, device=DEV)
    return wl, pw, canon, bits


@pytest.mark.parametrize("name,T", CASES, ids=[f"{n}-T{t}" for n, t in CASES])
def test_config_full_size(name, T):
    wl, pw, canon, bits = _prepared(name)
    op = {"swiglu": w4.OP_SWIGLU, "add": w4.OP_ADD}.get(wl.op, w4.OP_LINEAR)
    route = w4.route_name(w4.route_for(op, bits, T, pw.N, pw.K))
    print(f"case config={name} T={T} N={pw.N} K={pw.K} bits={bits} op={wl.op} route={route}", flush=True)
    x = wl.x[:T]
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    if wl.op == "swiglu":
        y = w4.linear_swiglu(xd, pw)
    elif wl.op == "add":
        y = w4.linear_add(xd, pw, torch.from_numpy(np.ascontiguousarray(wl.r[:T])).to(DEV))
    else:
        y = w4.linear(xd, pw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(T + 1000 * len(name))
    cols = np.sort(rng.choice(pw.N, NCOLS, replace=False))
    cols = np.unique(np.concatenate([cols, [0, pw.N - 1]]))  # first and last column too
    got = y[:, torch.from_numpy(cols).to(DEV)].cpu().numpy().astype(np.float64)
    if wl.op == "swiglu":
        g, u = canon
        ref = oracle.silu(oracle.linear_rows(x, *g, bits, cols)) * oracle.linear_rows(x, *u, bits, cols)
    else:
        ref = oracle.linear_rows(x, *canon, bits, cols)
        if wl.op == "add":
            ref = ref + wl.r[:T][:, cols].astype(np.float64)
    assert_close(got, ref, f"{name} T={T}")


FULL_CASES = [("decode", 1), ("decode", 4), ("batched", 64), ("swiglu", 16), ("prefill", 1024)]


@pytest.mark.parametrize("name,T", FULL_CASES, ids=[f"{n}-T{t}" for n, t in FULL_CASES])
def test_config_every_output(name, T):
    """The same configurations checked over every output element (the oracle over all N)."""
    wl, pw, canon, bits = _prepared(name)
    op = {"swiglu": w4.OP_SWIGLU, "add": w4.OP_ADD}.get(wl.op, w4.OP_LINEAR)
    route = w4.route_name(w4.route_for(op, bits, T, pw.N, pw.K))
    print(f"case config-all config={name} T={T} N={pw.N} K={pw.K} bits={bits} route={route}", flush=True)
    x = wl.x[:T]
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    if wl.op == "swiglu":
        y = w4.linear_swiglu(xd, pw)
        ref = oracle.swiglu(x, canon[0], canon[1], bits=bits)
    elif wl.op == "add":
        r = np.ascontiguousarray(wl.r[:T])
        y = w4.linear_add(xd, pw, torch.from_numpy(r).to(DEV))
        ref = oracle.linear_add(x, *canon, r, bits=bits)
    else:
        y = w4.linear(xd, pw)
        ref = oracle.linear(x, *canon, bits=bits)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy().astype(np.float64), ref, f"{name} T={T} all outputs")
