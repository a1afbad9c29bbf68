"""GPU tier: the grouped call (several packed matrices, 4- or 5-bit, over one activation, each
with its own output).  Each output must equal, bit for bit, the single-matrix launch of the
route the grouped call runs for that matrix (for T <= 64 and K <= 5120 the streaming route of
its width: same kernel, same summation order; otherwise the route w4_linear picks), and match
the fp64 oracle.  Small shapes
span ragged row tiles, a half k-block (K % 128 == 64) and every slice and ring mode of the
one-launch path (T <= 4, 5..8, 9..16, 17..32, 33..64) plus a width above it (one launch per
matrix); the full-size cases
are the two mixed-width input projections of the hybrid model the measurements come from
(4-bit 4096 + 5-bit 12288, 4-bit 7168 + 5-bit 7168, K = 5120) and the batched workload's two
4-bit parents, checked on sampled columns; between them they take one, two and three row tiles
per workgroup."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w4_groupwise_gemm_amd as w4
from synth import make_weights, make_activations
from gpu_util import assert_close, canon, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _single(xd, pw, T, K):
    """The single-matrix launch of the kernel the grouped call runs for this matrix."""
    if T <= 64 and K <= 5120:
        name = "mfma_stream_t16" if T <= 16 else "mfma_stream_t32" if T <= 32 else "mfma_stream_t64"
        rid = {w4.route_name(i): i for i in range(w4.route_count())}[name]
        return w4.linear_route(rid, w4.OP_LINEAR, xd, pw)
    return w4.linear(xd, pw)


def _weights(rng, specs, K):
    out = []
    for i, (N, bits) in enumerate(specs):
        scale = (0.0025, 0.01) if bits == 5 else (0.005, 0.02)
        out.append(make_weights(rng, f"p{i}", N, K, bits, ("uniform", 6, 9), scale))
    return out


SMALL = [((272, 4), (400, 5), (96, 4)), ((128, 5),), ((64, 4), (48, 5), (32, 4), (16, 5))]


@pytest.mark.parametrize("T", [1, 3, 4, 5, 8, 9, 16, 17, 24, 32, 33, 40, 64, 65])
@pytest.mark.parametrize("K", [704, 5120])
@pytest.mark.parametrize("specs", SMALL, ids=lambda s: "+".join(f"{n}b{b}" for n, b in s))
def test_grouped_matches_single_and_oracle(specs, K, T):
    rng = np.random.default_rng(T + K + 13 * len(specs))
    ws = _weights(rng, specs, K)
    x, _ = make_activations(rng, T, K, 1.0, 4)
    pws = [w4.pack_weight(*canon(w), b, device=DEV) for w, (_, b) in zip(ws, specs)]
    xd = torch.from_numpy(x).to(DEV)
    print(f"case grouped specs={specs} K={K} T={T}", flush=True)
    ys = w4.linear_grouped(xd, pws)
    singles = [_single(xd, pw, T, K) for pw in pws]
    torch.cuda.synchronize()
    for i, (y, y1, w, (_, b)) in enumerate(zip(ys, singles, ws, specs)):
        assert np.array_equal(to_np(y).view(np.uint16), to_np(y1).view(np.uint16)), (i, specs, K, T)
        assert_close(to_np(y), oracle.linear(x, *canon(w), bits=b), f"grouped p{i} T={T}")


def test_grouped_repeat_and_stream_order():
    """Back-to-back grouped calls on one stream with different widths and matrices: each result
    equals its single-matrix counterpart (no state carried between launches)."""
    rng = np.random.default_rng(99)
    K = 1024
    ws = _weights(rng, ((320, 4), (160, 5)), K)
    pws = [w4.pack_weight(*canon(w), b, device=DEV) for w, b in zip(ws, (4, 5))]
    for T in (16, 2, 7, 1, 12, 40, 20):
        x, _ = make_activations(rng, T, K, 1.0, 0)
        xd = torch.from_numpy(x).to(DEV)
        ys = w4.linear_grouped(xd, pws[::-1] if T % 2 else pws)
        ref = [_single(xd, pw, T, K) for pw in (pws[::-1] if T % 2 else pws)]
        torch.cuda.synchronize()
        for y, r in zip(ys, ref):
            assert np.array_equal(to_np(y).view(np.uint16), to_np(r).view(np.uint16)), T


# the two mixed-width projections (two row tiles per workgroup at T = 5..16: 512 and 448
# workgroups) and the batched workload's two 4-bit parents as a group (three row tiles: 236)
FULL = [((4096, 4), (12288, 5)), ((7168, 4), (7168, 5)), ((7168, 4), (4096, 4))]


@pytest.mark.parametrize("T", [1, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("specs", FULL, ids=lambda s: "+".join(f"{n}b{b}" for n, b in s))
def test_grouped_full_size(specs, T):
    K = 5120
    rng = np.random.default_rng(2024 + T)
    ws = _weights(rng, specs, K)
    x, _ = make_activations(rng, T, K, 1.0, 4)
    pws = [w4.pack_weight(*canon(w), b, device=DEV) for w, (_, b) in zip(ws, specs)]
    xd = torch.from_numpy(x).to(DEV)
    print(f"case grouped full specs={specs} T={T}", flush=True)
    ys = w4.linear_grouped(xd, pws)
    singles = [_single(xd, pw, T, K) for pw in pws]
    torch.cuda.synchronize()
    for i, (y, y1, w, (N, b)) in enumerate(zip(ys, singles, ws, specs)):
        assert np.array_equal(to_np(y).view(np.uint16), to_np(y1).view(np.uint16)), (i, specs, T)
        cols = np.unique(np.concatenate([np.random.default_rng(i + T).choice(N, 64, replace=False),
                                         [0, N - 1]]))
        got = to_np(y)[:, cols]
        assert_close(got, oracle.linear_rows(x, *canon(w), b, cols), f"grouped full p{i} T={T}")
