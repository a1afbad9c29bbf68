"""GPU tier: the A8 prefill route (int8 activations per 64 columns, int8 matrix-core steps).

* the quantised activations in the workspace equal the oracle's quantize_a8 bit for bit (codes
  and fp32 scales: both sides take the same fp32 decisions);
* every op's output against the oracle's A8 product (linear_a8: the same int8 activations in
  fp64) with the library's usual bounds, and against the exact product within the pages' 0.04
  relative L2 allowance for the route;
* ragged token counts, half-empty last k-blocks, odd tile counts, 4- and 5-bit codes;
* one quantisation serving two matrices (x = NULL), and NaN outputs for fractional zero-points.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w4_groupwise_gemm_amd as w4
from synth import make_weights, make_activations, make_residual, make_workload
from gpu_util import assert_close, canon, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PERM = [0, 4, 1, 5, 2, 6, 3, 7]  # byte order of each 8-column run in the workspace


def _unpack_ws(ws, T, K):
    raw = ws.cpu().numpy()
    q = raw[:T * K].view(np.int8).reshape(T, K // 8, 8)
    qn = np.empty_like(q)
    qn[:, :, PERM] = q
    off = (T * K + 15) // 16 * 16
    KB = (K + 127) // 128
    s = raw[off:off + KB * T * 2 * 4].view(np.float32).reshape(KB, T, 2)
    s = s.transpose(1, 0, 2).reshape(T, 2 * KB)[:, :K // 64]
    return qn.reshape(T, K), s


@pytest.mark.parametrize("T,K", [(1, 64), (5, 704), (33, 6144), (130, 1024)])
def test_quantised_activations_bitwise(T, K):
    rng = np.random.default_rng(T + K)
    x, _ = make_activations(rng, T, K, 1.0, 4)
    x[0, 64:128] = 0                   # an all-zero group (when K > 64)
    x[-1, :8] = [127, 0.5, 1.5, 2.5, -0.5, -1.5, 126.5, -3.25]  # ties, scale 1 if it is the max
    ws = w4.quantize_a8(torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    q, s = _unpack_ws(ws, T, K)
    q_ref, s_ref = oracle.quantize_a8(x)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)


def _case(N, K, T, bits, op, seed):
    rng = np.random.default_rng(seed)
    scale = (0.0025, 0.01) if bits == 5 else (0.005, 0.02)
    z = ("const", 16) if bits == 5 else ("uniform", 6, 9)
    ws = [make_weights(rng, "w", N, K, bits, z, scale)]
    if op == w4.OP_SWIGLU:
        ws.append(make_weights(rng, "u", N, K, bits, z, scale))
    x, _ = make_activations(rng, T, K, 0.5 if op == w4.OP_SWIGLU else 1.0, 0 if op == w4.OP_SWIGLU else 8)
    r = make_residual(rng, T, N)
    return ws, x, r


def _refs(ws, x, r, op, bits):
    """(the A8 route's own product, the exact product), fp64."""
    if op == w4.OP_SWIGLU:
        g8 = oracle.linear_a8(x, *canon(ws[0]), bits)
        u8 = oracle.linear_a8(x, *canon(ws[1]), bits)
        return oracle.silu(g8) * u8, oracle.swiglu(x, canon(ws[0]), canon(ws[1]), bits=bits)
    y8 = oracle.linear_a8(x, *canon(ws[0]), bits)
    y = oracle.linear(x, *canon(ws[0]), bits=bits)
    if op == w4.OP_ADD:
        return y8 + r.astype(np.float64), y + r.astype(np.float64)
    return y8, y


@pytest.mark.parametrize("op", [w4.OP_LINEAR, w4.OP_SWIGLU, w4.OP_ADD])
@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("N,K,T", [(272, 704, 1), (272, 704, 130), (336, 1024, 128), (160, 6144, 300)])
def test_a8_ops(N, K, T, bits, op):
    ws, x, r = _case(N, K, T, bits, op, seed=N + K + T + bits + 7 * op)
    pw = (w4.pack_pair(canon(ws[0]), canon(ws[1]), bits, device=DEV) if op == w4.OP_SWIGLU
          else w4.pack_weight(*canon(ws[0]), bits, device=DEV))
    xd = torch.from_numpy(x).to(DEV)
    print(f"case a8 op={op} bits={bits} T={T} N={N} K={K}", flush=True)
    if op == w4.OP_SWIGLU:
        y = w4.linear_swiglu_a8(xd, pw)
    elif op == w4.OP_ADD:
        y = w4.linear_add_a8(xd, pw, torch.from_numpy(r).to(DEV))
    else:
        y = w4.linear_a8(xd, pw)
    torch.cuda.synchronize()
    got = to_np(y).astype(np.float64)
    ref8, exact = _refs(ws, x, r, op, bits)
    assert_close(got, ref8, f"a8 op{op} b{bits} T{T} vs the A8 oracle")
    assert oracle.rel_l2(got, exact) <= 0.04


def test_a8_prefill_configuration():
    """The prefill workload (W5 LinearAdd, 5120 x 6144, outlier channels) at T = 1024 over every
    output, and at T = 4096 on sampled columns."""
    wl = make_workload("prefill")
    ws = wl.weights[0]
    pw = w4.pack_weight(*canon(ws), 5, device=DEV)
    for T in (1024, 4096):
        x = np.ascontiguousarray(wl.x[:T])
        r = np.ascontiguousarray(wl.r[:T])
        y = w4.linear_add_a8(torch.from_numpy(x).to(DEV), pw, torch.from_numpy(r).to(DEV))
        torch.cuda.synchronize()
        got = to_np(y).astype(np.float64)
        if T == 1024:
            cols = np.arange(ws.N)
        else:
            cols = np.unique(np.concatenate([np.random.default_rng(T).choice(ws.N, 128, replace=False), [0, ws.N - 1]]))
        q, s = oracle.quantize_a8(x)
        xa = q.astype(np.float64) * np.repeat(s.astype(np.float64), 64, axis=1)
        ref8 = oracle.linear_rows(xa, *canon(ws), 5, cols) + r[:, cols].astype(np.float64)
        exact = oracle.linear_rows(x, *canon(ws), 5, cols) + r[:, cols].astype(np.float64)
        print(f"case a8 prefill T={T}: rel_l2 vs exact {oracle.rel_l2(got[:, cols], exact):.4f}", flush=True)
        assert_close(got[:, cols], ref8, f"a8 prefill T={T}")
        assert oracle.rel_l2(got[:, cols], exact) <= 0.04


def test_a8_quantise_once_for_two_matrices():
    rng = np.random.default_rng(5)
    K, T = 1024, 96
    a = make_weights(rng, "a", 256, K, 4, ("uniform", 6, 9), (0.005, 0.02))
    b = make_weights(rng, "b", 512, K, 5, ("const", 16), (0.0025, 0.01))
    pa, pb = w4.pack_weight(*canon(a), 4, device=DEV), w4.pack_weight(*canon(b), 5, device=DEV)
    x, _ = make_activations(rng, T, K, 1.0, 8)
    xd = torch.from_numpy(x).to(DEV)
    ws = w4.quantize_a8(xd)
    ya = w4.linear_a8(None, pa, workspace=ws, T=T)
    yb = w4.linear_a8(None, pb, workspace=ws, T=T)
    za = w4.linear_a8(xd, pa)
    zb = w4.linear_a8(xd, pb)
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int16), za.view(torch.int16))
    assert torch.equal(yb.view(torch.int16), zb.view(torch.int16))


def test_a8_fractional_zero_points_give_nan():
    rng = np.random.default_rng(6)
    N, K, T = 256, 512, 8
    ws = make_weights(rng, "w", N, K, 4, ("uniform", 6, 9), (0.005, 0.02))
    z = ws.zeros.copy()
    z[130, 3] = np.float16(7.5)  # row 130: the second 128-row block
    pw = w4.pack_weight(ws.lo, ws.hi, ws.scales, z, 4, device=DEV)
    x, _ = make_activations(rng, T, K, 1.0, 0)
    y = to_np(w4.linear_a8(torch.from_numpy(x).to(DEV), pw)).astype(np.float64)
    assert np.all(np.isnan(y[:, 128:256]))
    ref8 = oracle.linear_a8(x, ws.lo, ws.hi, ws.scales, z, 4)
    assert_close(y[:, :128], ref8[:, :128], "integer zero-point block")
