"""GPU tier: the variants of the measured format on every route, against the fp64 oracle.

* groups of 32 and 128 columns per scale / zero-point (the pages use 64);
* bf16 activations, residuals and outputs (the pages' kernels run bf16 activations): every
  token row is carried into the fp16 kernels as X[t] * 2^-e_t, and the epilogue rounds to bf16;
  checked with the same bounds as the fp16 path (relative L2 <= 2e-3, element error <=
  1e-2 (1 + |y|)) against the oracle evaluated on the exact bf16 input values;
* bf16 rows far outside fp16's range (magnitudes near 1e6 and near 1e-6), which only the
  per-token power of two keeps exact.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w4_groupwise_gemm_amd as w4
from synth import make_weights, make_activations, make_activations_bf16, make_residual, bf16_bits
from gpu_util import assert_close, canon, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

ROUTE_TS = {
    "gemv_exact_t": (1, 4),
    "mfma_stream_t16": (1, 5, 9, 16),
    "mfma_narrow_t32": (3, 32),
    "mfma_narrow_t64": (33, 64),
    "mfma_wide": (1, 129),
    "mfma_splitk_t32": (7, 32),
    "mfma_narrow_tiled": (65, 130),
    "mfma_stream_t32": (17, 32),
    "mfma_stream_t64": (33, 64),
    "mfma_bal_t32": (5, 32),
    "mfma_bal_t64": (33, 64),
    "mfma_reg_t16": (1, 16),
    "mfma_reg_t32": (5, 32),
    "mfma_reg_t64": (33, 64),
    "mfma_reg32_t32": (5, 32),
    "mfma_reg32_t64": (33, 64),
}


def route_ids():
    return {w4.route_name(i): i for i in range(w4.route_count())}


def _params():
    return [(route, op, bits, T) for route, ts in ROUTE_TS.items()
            for op in (w4.OP_LINEAR, w4.OP_SWIGLU, w4.OP_ADD) for bits in (4, 5) for T in ts]


def _weights(rng, N, K, bits, op, group):
    scale = (0.0025, 0.01) if bits == 5 else (0.005, 0.02)
    ws = [make_weights(rng, "w", N, K, bits, ("uniform", 6, 9), scale, group=group)]
    if op == w4.OP_SWIGLU:
        ws.append(make_weights(rng, "u", N, K, bits, ("uniform", 6, 9), scale, group=group))
        pw = w4.pack_pair(canon(ws[0]), canon(ws[1]), bits, device=DEV, group=group)
    else:
        pw = w4.pack_weight(*canon(ws[0]), bits, device=DEV, group=group)
    return ws, pw


def _oracle(ws, x64, r64, op, bits, group):
    if op == w4.OP_SWIGLU:
        return oracle.swiglu(x64, canon(ws[0]), canon(ws[1]), bits=bits, group=group)
    y = oracle.linear(x64, *canon(ws[0]), bits=bits, group=group)
    return y + r64 if op == w4.OP_ADD else y


@pytest.mark.parametrize("group,K", [(32, 704), (32, 768), (128, 768)])
@pytest.mark.parametrize("route,op,bits,T", _params(), ids=lambda v: str(v))
def test_group_sizes(route, op, bits, T, group, K):
    N = 272
    rng = np.random.default_rng(N + K + T + 7 * bits + 31 * op + group)
    ws, pw = _weights(rng, N, K, bits, op, group)
    x, _ = make_activations(rng, T, K, 0.5 if op == w4.OP_SWIGLU else 1.0, 0 if op == w4.OP_SWIGLU else 4)
    r = make_residual(rng, T, N)
    print(f"case group={group} route={route} op={op} bits={bits} T={T} K={K}", flush=True)
    y = w4.linear_route(route_ids()[route], op, torch.from_numpy(x).to(DEV), pw,
                        residual=torch.from_numpy(r).to(DEV) if op == w4.OP_ADD else None)
    torch.cuda.synchronize()
    ref = _oracle(ws, x.astype(np.float64), r.astype(np.float64), op, bits, group)
    assert_close(to_np(y), ref, f"group {group} {route} op{op} b{bits} T{T} K{K}")


def _bf16_dev(bits_u16):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(DEV).view(torch.bfloat16)


def _bf16_np(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("route,op,bits,T", _params(), ids=lambda v: str(v))
def test_bf16_activations(route, op, bits, T):
    N, K = 272, 704
    rng = np.random.default_rng(N + K + T + 7 * bits + 31 * op + 5)
    ws, pw = _weights(rng, N, K, bits, op, 64)
    xb, _ = make_activations_bf16(rng, T, K, 0.5 if op == w4.OP_SWIGLU else 1.0,
                                  0 if op == w4.OP_SWIGLU else 4)
    rb = bf16_bits(rng.standard_normal((T, N)).astype(np.float32))
    print(f"case bf16 route={route} op={op} bits={bits} T={T} K={K}", flush=True)
    y = w4.linear_route_bf16(route_ids()[route], op, _bf16_dev(xb), pw,
                             residual=_bf16_dev(rb) if op == w4.OP_ADD else None)
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16
    got = oracle.bf16_value(_bf16_np(y))
    ref = _oracle(ws, oracle.bf16_value(xb), oracle.bf16_value(rb), op, bits, 64)
    assert_close(got, ref, f"bf16 {route} op{op} b{bits} T{T}")


@pytest.mark.parametrize("route", sorted(ROUTE_TS))
def test_bf16_with_group_32(route):
    N, K, bits = 272, 768, 5
    T = ROUTE_TS[route][-1]
    rng = np.random.default_rng(77)
    ws, pw = _weights(rng, N, K, bits, w4.OP_LINEAR, 32)
    xb, _ = make_activations_bf16(rng, T, K, 1.0, 4)
    y = w4.linear_route_bf16(route_ids()[route], w4.OP_LINEAR, _bf16_dev(xb), pw)
    torch.cuda.synchronize()
    ref = _oracle(ws, oracle.bf16_value(xb), None, w4.OP_LINEAR, bits, 32)
    assert_close(oracle.bf16_value(_bf16_np(y)), ref, f"bf16 group 32 {route}")


@pytest.mark.parametrize("route", sorted(ROUTE_TS))
def test_bf16_rows_outside_fp16_range(route):
    """Token rows scaled by 2^20 (|x| up to ~4e6, past fp16's 65504) and by 2^-20 (|x| near
    1e-6, fp16 subnormals) next to an ordinary row: each row takes its own power of two."""
    N, K, bits = 96, 512, 4
    T = max(3, ROUTE_TS[route][0])
    rng = np.random.default_rng(88)
    ws, pw = _weights(rng, N, K, bits, w4.OP_LINEAR, 64)
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[0] *= np.float32(2.0 ** 20)
    x[1] *= np.float32(2.0 ** -20)
    xb = bf16_bits(x)
    y = w4.linear_route_bf16(route_ids()[route], w4.OP_LINEAR, _bf16_dev(xb), pw)
    torch.cuda.synchronize()
    got = oracle.bf16_value(_bf16_np(y))
    ref = _oracle(ws, oracle.bf16_value(xb), None, w4.OP_LINEAR, bits, 64)
    assert_close(got, ref, f"bf16 rows outside fp16 range {route}")
    # each row against its own magnitude (a wrong power of two would be off by a factor of two
    # or more): rounding to bf16 moves an element by at most 2^-9 of itself, the fp16 weights
    # add about 3.5e-4, so a row's relative L2 error stays below 2^-9 + 1e-3
    for t in range(T):
        rel = oracle.rel_l2(got[t], ref[t])
        assert rel <= 2.0 ** -9 + 1e-3, (route, t, rel)


def test_bf16_public_calls_match_their_route():
    """w4_linear_bf16 / _swiglu_bf16 / _add_bf16 run the route w4_route_for names (bitwise)."""
    N, K = 256, 512
    rng = np.random.default_rng(99)
    for op in (w4.OP_LINEAR, w4.OP_SWIGLU, w4.OP_ADD):
        ws, pw = _weights(rng, N, K, 4, op, 64)
        for T in (1, 4, 16, 24, 64, 200):
            xb, _ = make_activations_bf16(rng, T, K, 1.0, 2)
            rb = bf16_bits(rng.standard_normal((T, N)).astype(np.float32))
            xd, rd = _bf16_dev(xb), _bf16_dev(rb)
            if op == w4.OP_SWIGLU:
                y = w4.linear_swiglu_bf16(xd, pw)
            elif op == w4.OP_ADD:
                y = w4.linear_add_bf16(xd, pw, rd)
            else:
                y = w4.linear_bf16(xd, pw)
            rid = w4.route_for(op, 4, T, N, K)
            y2 = w4.linear_route_bf16(rid, op, xd, pw, residual=rd if op == w4.OP_ADD else None)
            assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), (op, T)


# The 32-row register ring with K split over workgroups (640 rows: 20 tile pairs, four K
# slices): groups of 32 and 128 columns, and bf16 activations, residuals and outputs through the
# split's last-workgroup epilogue.
@pytest.mark.parametrize("route,T", [("mfma_reg32_t32", 24), ("mfma_reg32_t64", 64)])
@pytest.mark.parametrize("group,K", [(32, 12352), (128, 16384)])
def test_k_split_group_sizes(route, T, group, K):
    N, bits = 640, 5
    rng = np.random.default_rng(K + T + group)
    ws, pw = _weights(rng, N, K, bits, w4.OP_ADD, group)
    x, _ = make_activations(rng, T, K, 1.0, 4)
    r = make_residual(rng, T, N)
    print(f"case split group={group} route={route} T={T} K={K}", flush=True)
    y = w4.linear_route(route_ids()[route], w4.OP_ADD, torch.from_numpy(x).to(DEV), pw,
                        residual=torch.from_numpy(r).to(DEV))
    torch.cuda.synchronize()
    ref = _oracle(ws, x.astype(np.float64), r.astype(np.float64), w4.OP_ADD, bits, group)
    assert_close(to_np(y), ref, f"split group {group} {route} T{T} K{K}")


@pytest.mark.parametrize("op", [w4.OP_LINEAR, w4.OP_SWIGLU, w4.OP_ADD])
def test_k_split_bf16(op):
    N, K, bits, T = 640, 12352, 4, 32
    rng = np.random.default_rng(300 + op)
    ws, pw = _weights(rng, N, K, bits, op, 64)
    xb, _ = make_activations_bf16(rng, T, K, 0.5 if op == w4.OP_SWIGLU else 1.0, 0)
    rb = bf16_bits(rng.standard_normal((T, N)).astype(np.float32))
    print(f"case split bf16 op={op}", flush=True)
    y = w4.linear_route_bf16(route_ids()["mfma_reg32_t32"], op, _bf16_dev(xb), pw,
                             residual=_bf16_dev(rb) if op == w4.OP_ADD else None)
    torch.cuda.synchronize()
    got = oracle.bf16_value(_bf16_np(y))
    ref = _oracle(ws, oracle.bf16_value(xb), oracle.bf16_value(rb), op, bits, 64)
    # (the SwiGLU pair beyond K = 5120 is held to the relative L2 bound)
    assert_close(got, ref, f"split bf16 op{op}", elem=op != w4.OP_SWIGLU)
