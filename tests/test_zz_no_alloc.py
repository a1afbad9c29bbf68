"""GPU tier: the allocation-free bf16 linear call (w4_linear_bf16_noalloc, static device
scratch) through the C ABI, against the same call with a caller workspace (w4_linear_bf16:
the same kernels, so bit-identical) and against the fp64 oracle, on two calls in a row, the
second with a smaller input (the scratch keeps the first call's contents)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import w4_groupwise_gemm_amd as w4
from synth import make_weights, make_activations_bf16
from gpu_util import assert_close, canon

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bf16_dev(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(DEV).view(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _run(L, x, pw, T, N, K, stream):
    """(no-alloc output, workspace-call output) through the C ABI."""
    y0 = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    y1 = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(w4.bf16_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    args = (x.data_ptr(), pw.w.data_ptr(), pw.scales.data_ptr(), pw.zeros.data_ptr())
    st = L.w4_linear_bf16_noalloc(*args, T, N, K, pw.bits, pw.group, y0.data_ptr(), stream)
    assert st == 0, w4.status_str(st)
    st = L.w4_linear_bf16(*args, T, N, K, pw.bits, pw.group, y1.data_ptr(), ws.data_ptr(),
                          ws.numel(), stream)
    assert st == 0, w4.status_str(st)
    torch.cuda.synchronize()
    return y0, y1


@pytest.mark.parametrize("bits", [4, 5])
def test_noalloc_matches_workspace_call(bits):
    L = w4.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rng = np.random.default_rng(123 + bits)
    scale = (0.0025, 0.01) if bits == 5 else (0.005, 0.02)
    # first call: 1024 tokens x K = 5120 (10 MiB of scratch); second: 3 tokens x K = 1024
    for (T, N, K) in ((1024, 1024, 5120), (3, 512, 1024)):
        print(f"case noalloc bits={bits} T={T} N={N} K={K}", flush=True)
        ws = make_weights(rng, "w", N, K, bits, ("uniform", 6, 9), scale)
        pw = w4.pack_weight(*canon(ws), bits, device=DEV)
        xb, _ = make_activations_bf16(rng, T, K, 1.0, 4)
        y0, y1 = _run(L, _bf16_dev(xb), pw, T, N, K, stream)
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), (T, N, K)
        cols = np.unique(np.concatenate([rng.choice(N, 128, replace=False), [0, N - 1]]))
        ref = oracle.linear_rows(oracle.bf16_value(xb), *canon(ws), bits, cols)
        assert_close(oracle.bf16_value(_bits(y0))[:, cols], ref, f"noalloc T={T} K={K}")


def test_noalloc_rejects_oversize():
    L = w4.lib()
    T, N, K = 4096, 16, 6144  # 48 MiB of workspace needed
    assert w4.bf16_workspace_bytes(T, K) > w4.SCRATCH_BYTES
    x = torch.zeros((T, K), dtype=torch.bfloat16, device=DEV)
    pw = w4.pack_weight(*canon(make_weights(np.random.default_rng(1), "w", N, K, 4, ("const", 8),
                                            (0.005, 0.02))), 4, device=DEV)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    st = L.w4_linear_bf16_noalloc(x.data_ptr(), pw.w.data_ptr(), pw.scales.data_ptr(),
                                  pw.zeros.data_ptr(), T, N, K, 4, 64, y.data_ptr(), None)
    assert st == -8
