"""CPU tier: the binding rejects tensors the library cannot check (it receives bare pointers)
with ValueError before any launch: wrong device, element type, shape or layout of the
activations, the residual, the output and the packed weights."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import w4_groupwise_gemm_amd as w4

CPU = torch.device("cpu")


def _pw(N=32, K=128, bits=4, pair=False, device=CPU):
    rows = 2 * N if pair else N
    nw, nsz = w4.packed_bytes(rows, K, bits), w4.packed_sz_bytes(rows, K)
    return w4.PackedWeight(torch.zeros(nw, dtype=torch.uint8, device=device),
                           torch.zeros(nsz // 2, dtype=torch.int16, device=device),
                           torch.zeros(nsz // 2, dtype=torch.int16, device=device), N, K, bits, pair)


def test_check_tensor_cases():
    good = torch.zeros((3, 8), dtype=torch.float16)
    w4._check_tensor(good, "t", (3, 8), torch.float16, CPU)
    with pytest.raises(ValueError, match="float16"):
        w4._check_tensor(good.float(), "t", (3, 8), torch.float16, CPU)
    with pytest.raises(ValueError, match="shape"):
        w4._check_tensor(good, "t", (3, 7), torch.float16, CPU)
    with pytest.raises(ValueError, match="contiguous"):
        w4._check_tensor(torch.zeros((8, 3), dtype=torch.float16).t(), "t", (3, 8), torch.float16, CPU)
    with pytest.raises(ValueError, match="expected"):
        w4._check_tensor(good.to("meta"), "t", (3, 8), torch.float16, CPU)
    with pytest.raises(ValueError, match="torch tensor"):
        w4._check_tensor(np.zeros((3, 8), np.float16), "t", (3, 8), torch.float16, CPU)


def test_residual_and_out_checks():
    like = torch.zeros((4, 128), dtype=torch.float16)
    w4._check_residual(torch.zeros((4, 32), dtype=torch.float16), 4, 32, like)
    for bad in (torch.zeros((4, 32), dtype=torch.float32), torch.zeros((4, 16), dtype=torch.float16),
                torch.zeros((32, 4), dtype=torch.float16).t(), torch.zeros((4, 32), dtype=torch.float16, device="meta")):
        with pytest.raises(ValueError):
            w4._check_residual(bad, 4, 32, like)
        with pytest.raises(ValueError):
            w4._out(bad, 4, 32, like)


def test_weight_checks():
    w4._check_weight(_pw(), CPU)
    w4._check_weight(_pw(pair=True), CPU)
    short = _pw()
    short.w = short.w[:-16]
    with pytest.raises(ValueError, match="packed codes"):
        w4._check_weight(short, CPU)
    wrong = _pw()
    wrong.scales = wrong.scales.float()
    with pytest.raises(ValueError, match="packed scales"):
        w4._check_weight(wrong, CPU)
    with pytest.raises(ValueError, match="expected"):
        w4._check_weight(_pw(device="meta"), CPU)


def test_host_activations_rejected_before_launch():
    x = torch.zeros((2, 128), dtype=torch.float16)  # host memory: never handed to a kernel
    pw = _pw()
    for call in (lambda: w4.linear(x, pw), lambda: w4.linear_add(x, pw, torch.zeros((2, 32), dtype=torch.float16)),
                 lambda: w4.linear_route(1, w4.OP_LINEAR, x, pw), lambda: w4.linear_grouped(x, [pw])):
        with pytest.raises(ValueError):
            call()
    with pytest.raises(ValueError, match="pair"):
        w4.linear(x, _pw(pair=True))
    with pytest.raises(ValueError, match="pair"):
        w4.linear_swiglu(x, pw)
