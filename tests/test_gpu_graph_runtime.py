"""GPU tier: HIP-graph capture and replay of every op, in-place LinearAdd, guard bands,
padding rows that must never be read, and the single-HIP-runtime check."""
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


def _setup(op, N, K, T, bits, seed):
    rng = np.random.default_rng(seed)
    scale = (0.0025, 0.01) if bits == 5 else (0.005, 0.02)
    ws = [make_weights(rng, "w", N, K, bits, ("uniform", 6, 9), scale)]
    if op == w4.OP_SWIGLU:
        ws.append(make_weights(rng, "u", N, K, bits, ("uniform", 6, 9), scale))
        pw = w4.pack_pair(canon(ws[0]), canon(ws[1]), bits, device=DEV)
    else:
        pw = w4.pack_weight(*canon(ws[0]), bits, device=DEV)
    x, _ = make_activations(rng, T, K, 1.0, 2)
    r = make_residual(rng, T, N)
    return ws, pw, torch.from_numpy(x).to(DEV), torch.from_numpy(r).to(DEV)


def _call(op, x, pw, r, out):
    if op == w4.OP_SWIGLU:
        return w4.linear_swiglu(x, pw, out=out)
    if op == w4.OP_ADD:
        return w4.linear_add(x, pw, r, out=out)
    return w4.linear(x, pw, out=out)


@pytest.mark.parametrize("op", [w4.OP_LINEAR, w4.OP_SWIGLU, w4.OP_ADD])
@pytest.mark.parametrize("T", [1, 4, 16, 24, 40, 200])
def test_graph_replays_match_eager(op, T):
    N, K, bits = 256, 1024, 4 if op != w4.OP_ADD else 5
    ws, pw, x, r = _setup(op, N, K, T, bits, seed=T + 10 * op)
    eager = _call(op, x, pw, r, torch.empty((T, N), dtype=torch.float16, device=DEV)).clone()
    static_out = torch.empty((T, N), dtype=torch.float16, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(op, x, pw, r, static_out)
    for rep in range(4):
        # the program's own eager work between replays
        static_out.fill_(float("nan"))
        junk = torch.randn(4096, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(static_out.view(torch.int16), eager.view(torch.int16)), (op, T, rep)
        del junk


@pytest.mark.parametrize("T", [1, 3, 16, 33, 300])
def test_linear_add_in_place(T):
    """out == residual: each element is read once and written once (no double add)."""
    N, K, bits = 192, 768, 5
    ws, pw, x, r = _setup(w4.OP_ADD, N, K, T, bits, seed=77 + T)
    r0 = r.clone()
    out = w4.linear_add(x, pw, r, out=r)
    torch.cuda.synchronize()
    assert out.data_ptr() == r.data_ptr()
    ref = oracle.linear_add(to_np(x), *canon(ws[0]), to_np(r0), bits=bits)
    assert_close(to_np(r), ref, "in-place LinearAdd")
    # and bitwise equal to the out-of-place result
    out2 = w4.linear_add(x, pw, r0)
    assert torch.equal(out2.view(torch.int16), r.view(torch.int16))


@pytest.mark.parametrize("op", [w4.OP_LINEAR, w4.OP_SWIGLU, w4.OP_ADD])
@pytest.mark.parametrize("T", [1, 5, 17, 64, 130])
def test_padding_rows_and_guard_bands(op, T):
    """Rows of x beyond T are NaN and must not be read; bytes around out must not change."""
    N, K, bits = 128, 640, 4
    ws, pw, x, r = _setup(op, N, K, T, bits, seed=5 * T + op)
    xbig = torch.full((T + 37, K), float("nan"), dtype=torch.float16, device=DEV)
    xbig[:T] = x
    guard = 4096
    buf = torch.full((guard + T * N + guard,), 0x7BCD, dtype=torch.int16, device=DEV)
    out = buf[guard:guard + T * N].view(torch.float16).view(T, N)
    y = _call(op, xbig[:T], pw, r, out)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:guard] == 0x7BCD) and np.all(b[guard + T * N:] == 0x7BCD)
    assert np.all(np.isfinite(to_np(y).astype(np.float64)))


def test_single_hip_runtime_mapped():
    w4.lib()
    torch.zeros(1, device=DEV)
    maps = open("/proc/self/maps").read().splitlines()
    paths = {ln.split()[-1] for ln in maps if "libamdhip64" in ln}
    assert len(paths) == 1, paths
