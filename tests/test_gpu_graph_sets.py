"""GPU tier: per-verify-width graph sets (w4_graph_set_*, VerifyGraphs).

A small decode step -- a grouped mixed-width input projection, a SwiGLU pair, and a LinearAdd
fed by the SwiGLU output -- is recorded once per width T in {1, 2, 4, 8} and replayed several
times, with new activations written between replays by the program's own eager work.  Every
replay must equal the same calls launched eagerly, bit for bit (same kernels, same inputs)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import w4_groupwise_gemm_amd as w4
from synth import make_weights, make_activations
from gpu_util import canon

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
WIDTHS = (1, 2, 4, 8)
K, NG, ND = 1024, 512, 1024


def _weights():
    rng = np.random.default_rng(2024)
    a = make_weights(rng, "a", 1024, K, 4, ("uniform", 6, 9), (0.005, 0.02))
    b = make_weights(rng, "b", 2048, K, 5, ("const", 16), (0.0025, 0.01))
    g = make_weights(rng, "g", NG, K, 4, ("uniform", 6, 9), (0.005, 0.02))
    u = make_weights(rng, "u", NG, K, 4, ("uniform", 6, 9), (0.005, 0.02))
    d = make_weights(rng, "d", ND, NG, 4, ("uniform", 6, 9), (0.005, 0.02))
    return (w4.pack_weight(*canon(a), 4, device=DEV), w4.pack_weight(*canon(b), 5, device=DEV),
            w4.pack_pair(canon(g), canon(u), 4, device=DEV), w4.pack_weight(*canon(d), 4, device=DEV))


def _buffers(T):
    f = dict(dtype=torch.float16, device=DEV)
    return {"x": torch.zeros((T, K), **f), "qa": torch.empty((T, 1024), **f), "qb": torch.empty((T, 2048), **f),
            "h": torch.empty((T, NG), **f), "r": torch.zeros((T, ND), **f), "y": torch.empty((T, ND), **f)}


def _step(W, B, stream):
    pa, pb, pp, pd = W
    w4.linear_grouped(B["x"], [pa, pb], outs=[B["qa"], B["qb"]], stream=stream)
    w4.linear_swiglu(B["x"], pp, out=B["h"], stream=stream)
    w4.linear_add(B["h"], pd, B["r"], out=B["y"], stream=stream)


def test_graph_replays_match_eager():
    W = _weights()
    graphs = w4.VerifyGraphs()
    rng = np.random.default_rng(7)
    bufs = {T: _buffers(T) for T in WIDTHS}
    for T in WIDTHS:
        graphs.record(T, lambda T, T0=T: _step(W, bufs[T0], graphs.stream))
        assert graphs.recorded(T)
    for rep in range(3):
        for T in WIDTHS:
            B = bufs[T]
            x, _ = make_activations(rng, T, K, 0.5, 2)
            r = rng.standard_normal((T, ND)).astype(np.float16)
            B["x"].copy_(torch.from_numpy(x))
            B["r"].copy_(torch.from_numpy(r))
            torch.cuda.synchronize()
            print(f"case graph-set replay={rep} T={T}", flush=True)
            graphs.run(T)
            graphs.stream.synchronize()
            got = {k: B[k].clone() for k in ("qa", "qb", "h", "y")}
            # the same calls, eagerly, on fresh buffers holding the same inputs
            E = _buffers(T)
            E["x"].copy_(B["x"])
            E["r"].copy_(B["r"])
            _step(W, E, None)
            torch.cuda.synchronize()
            for k in got:
                assert torch.equal(got[k].view(torch.int16), E[k].view(torch.int16)), (rep, T, k)
    graphs.close()


def test_graph_set_errors():
    graphs = w4.VerifyGraphs()
    with pytest.raises(KeyError):
        graphs.run(3)
    W = _weights()
    B = _buffers(2)
    graphs.record(2, lambda T: _step(W, B, graphs.stream))
    with pytest.raises(w4.W4Error):  # a width is recorded once
        graphs.record(2, lambda T: _step(W, B, graphs.stream))
    graphs.run(2)
    graphs.stream.synchronize()
    graphs.close()
