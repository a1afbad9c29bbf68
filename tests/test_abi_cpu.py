"""CPU tier: the C-ABI library loads, exports what the header declares, validates arguments
synchronously (no device work) and repacks bit-exactly against an independent layout model."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import w4_groupwise_gemm_amd as w4
from synth import make_weights, pack_canonical
from layout_spec import spec_pack, spec_unpack

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4gemm.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = w4.lib()
    names = header_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(w4.EXPORTS)


def test_layout_version_and_status_strings():
    assert w4.layout_version() == 1
    for st in range(0, -9, -1):
        assert w4.status_str(st) and w4.status_str(st) != "unknown status"
    assert w4.status_str(-99) == "unknown status"


def test_route_table_domains_cover_every_width():
    n = w4.route_count()
    assert n >= 5
    names = [w4.route_name(i) for i in range(n)]
    assert len(set(names)) == n and all(names)
    assert w4.route_name(n) is None and w4.route_name(-1) is None
    for op in (w4.OP_LINEAR, w4.OP_SWIGLU, w4.OP_ADD):
        for bits in (4, 5):
            for K in (512, 5120, 6144, 17408):
                for T in list(range(1, 130)) + [255, 256, 1000, 1024, 1025, 4096, 65536]:
                    r = w4.route_for(op, bits, T, 4096, K)
                    assert 0 <= r < n
                    lo, hi = w4.route_domain(r)
                    assert lo <= T <= hi, (op, bits, T, K, r)


@pytest.mark.parametrize("op,bits,T,N,K,route", [
    # K <= 5120, single matrices: streaming to 16 tokens, its 32-row ring to 32, its 64-row ring
    # to 64 (4-bit); 5-bit codes take the register ring at 5-16 and 33-48 tokens
    (0, 4, 16, 12288, 5120, "mfma_stream_t16"), (0, 4, 17, 12288, 5120, "mfma_stream_t32"),
    (2, 4, 64, 12288, 5120, "mfma_stream_t64"), (0, 5, 4, 12288, 5120, "mfma_stream_t16"),
    (0, 5, 5, 12288, 5120, "mfma_reg_t16"), (0, 5, 16, 12288, 5120, "mfma_reg_t16"),
    (0, 5, 17, 12288, 5120, "mfma_stream_t32"), (0, 5, 33, 12288, 5120, "mfma_reg_t64"),
    (0, 5, 48, 12288, 5120, "mfma_reg_t64"), (0, 5, 49, 12288, 5120, "mfma_narrow_t64"),
    # the SwiGLU pair at K <= 5120: streaming throughout with at most one pair per compute unit;
    # otherwise streaming to 8 tokens, then the register ring (its 32-token instance from 9
    # tokens with three or more pairs per compute unit)
    (1, 4, 16, 4096, 5120, "mfma_stream_t16"), (1, 4, 32, 4096, 5120, "mfma_stream_t32"),
    (1, 4, 64, 4096, 5120, "mfma_stream_t64"), (1, 4, 8, 17408, 5120, "mfma_stream_t16"),
    (1, 4, 9, 17408, 5120, "mfma_reg_t32"), (1, 4, 32, 17408, 5120, "mfma_reg_t32"),
    (1, 4, 33, 17408, 5120, "mfma_reg_t64"), (1, 4, 64, 17408, 5120, "mfma_reg_t64"),
    (1, 5, 9, 8192, 5120, "mfma_reg_t16"), (1, 5, 17, 8192, 5120, "mfma_reg_t32"),
    (1, 5, 48, 8192, 5120, "mfma_reg_t64"), (1, 5, 49, 8192, 5120, "mfma_bal_t64"),
    # K > 5120: streaming to 4 tokens (the 16-row register ring from the first token beyond
    # K = 8192), the 16-row register ring to 12 (16 below K = 12288), the 32-row ring beyond,
    # and from the first token beyond K = 16384
    (0, 5, 4, 5120, 6144, "mfma_stream_t16"), (0, 4, 4, 5120, 8192, "mfma_stream_t16"),
    (0, 5, 1, 5120, 12288, "mfma_reg_t16"), (2, 4, 4, 5120, 17408, "mfma_reg32_t32"),
    (0, 4, 1, 5120, 17408, "mfma_reg32_t32"), (0, 5, 16, 5120, 16384, "mfma_reg32_t32"),
    (0, 5, 4, 5120, 16384, "mfma_reg_t16"),
    (2, 5, 5, 5120, 6144, "mfma_reg_t16"), (0, 4, 16, 5120, 8192, "mfma_reg_t16"),
    (0, 5, 12, 5120, 12288, "mfma_reg_t16"), (0, 5, 13, 5120, 12288, "mfma_reg32_t32"),
    (0, 5, 17, 5120, 17408, "mfma_reg32_t32"), (2, 5, 24, 5120, 6144, "mfma_reg32_t32"),
    (0, 4, 32, 5120, 8192, "mfma_reg32_t32"), (0, 4, 33, 5120, 8192, "mfma_reg32_t64"),
    (0, 5, 64, 5120, 12288, "mfma_reg32_t64"),
    # the SwiGLU pair at K > 5120 (no measured shape): streaming to 16, narrow beyond
    (1, 5, 16, 5120, 6144, "mfma_stream_t16"), (1, 5, 17, 5120, 6144, "mfma_narrow_t32"),
])
def test_route_choice_follows_measured_crossovers(op, bits, T, N, K, route):
    assert w4.route_name(w4.route_for(op, bits, T, N, K)) == route


def test_route_for_rejects_bad_shapes():
    assert w4.route_for(7, 4, 1, 256, 512) == -2
    assert w4.route_for(0, 3, 1, 256, 512) == -2
    assert w4.route_for(0, 4, 1, 250, 512) == -1
    assert w4.route_for(0, 4, 1, 256, 500) == -1
    assert w4.route_for(0, 4, -1, 256, 512) == -1


# ---- synchronous validation: fake addresses are fine because nothing touches the device

def _call(fn, x=0x10000, w=0x20000000, s=0x30000000, z=0x40000000, T=4, N=256, K=512, bits=4,
          group=64, out=0x50000000, res=None):
    L = w4.lib()
    if fn == "add":
        return L.w4_linear_add(x, w, s, z, res if res is not None else 0x60000000, T, N, K, bits,
                               group, out, None)
    if fn == "swiglu":
        return L.w4_linear_swiglu(x, w, s, z, T, N, K, bits, group, out, None)
    return L.w4_linear(x, w, s, z, T, N, K, bits, group, out, None)


@pytest.mark.parametrize("fn", ["linear", "swiglu", "add"])
def test_validation_errors(fn):
    assert _call(fn, bits=3) == -2
    assert _call(fn, bits=8) == -2
    assert _call(fn, group=16) == -2
    assert _call(fn, group=48) == -2
    assert _call(fn, group=128, K=320) == -1   # groups of 128 need K % 128 == 0
    # groups of 32 and 128 pass validation (no GPU here: the device check is what fails)
    assert _call(fn, group=32) == -6
    assert _call(fn, group=128) == -6
    assert _call(fn, N=250) == -1
    assert _call(fn, N=0) == -1
    assert _call(fn, K=500) == -1
    assert _call(fn, K=0) == -1
    assert _call(fn, T=-1) == -1
    assert _call(fn, x=0) == -1
    assert _call(fn, w=0) == -1
    assert _call(fn, s=0) == -1
    assert _call(fn, z=0) == -1
    assert _call(fn, out=0) == -1
    assert _call(fn, x=0x10008) == -3
    assert _call(fn, w=0x20000004) == -3
    assert _call(fn, out=0x50000002) == -3
    # out overlapping x / w / scales
    assert _call(fn, out=0x10000 + 16) == -4
    assert _call(fn, out=0x20000000 + 1024) == -4
    assert _call(fn, out=0x30000000 + 16) == -4
    # T == 0 is a successful no-op, even with null pointers
    assert _call(fn, T=0, x=0, w=0, s=0, z=0, out=0) == 0


def test_linear_add_aliasing_rules():
    # out == residual exactly is allowed (validation passes; no GPU here so the device check
    # is what fails) -- partial overlap is an alias error
    assert _call("add", res=0x50000000 + 16) == -4
    assert _call("add", res=0) == -1
    assert _call("add", res=0x60000008) == -3


def test_forced_route_outside_domain():
    L = w4.lib()
    args = (0x10000, 0x20000000, 0x30000000, 0x40000000, None)
    n = w4.route_count()
    assert L.w4_linear_route(n, 0, *args, 4, 256, 512, 4, 64, 0x50000000, None) == -5
    assert L.w4_linear_route(-1, 0, *args, 4, 256, 512, 4, 64, 0x50000000, None) == -5
    for r in range(n):
        lo, hi = w4.route_domain(r)
        if hi < 1 << 24:
            assert L.w4_linear_route(r, 0, *args, hi + 1, 256, 512, 4, 64, 0x50000000, None) == -5


def test_packed_sizes():
    assert w4.packed_bytes(256, 512, 4) == 256 * 512 // 2
    assert w4.packed_bytes(256, 512, 5) == 256 * 512 * 5 // 8
    assert w4.packed_bytes(16, 64, 4) == 1024                 # half-empty k-block is padded
    assert w4.packed_sz_bytes(256, 512) == 256 * 512 // 64 * 2
    assert w4.packed_sz_bytes(16, 64) == 16 * 2 * 2
    assert w4.packed_bytes(250, 512, 4) == 0
    assert w4.packed_bytes(256, 500, 4) == 0
    assert w4.packed_bytes(256, 512, 6) == 0
    assert w4.packed_bytes(256, 512, 4) == w4.lib().w4_packed_bytes(256, 512, 4, 64)
    assert w4.lib().w4_packed_bytes(256, 512, 4, 16) == 0
    # codes do not depend on the group size; scales / zeros: one pair per row and 128 columns,
    # two for groups of 32
    assert w4.packed_bytes(256, 512, 4, 32) == w4.packed_bytes(256, 512, 4, 128) == 256 * 512 // 2
    assert w4.packed_sz_bytes(256, 512, 32) == 2 * w4.packed_sz_bytes(256, 512, 64)
    assert w4.packed_sz_bytes(256, 512, 128) == w4.packed_sz_bytes(256, 512, 64)
    assert w4.packed_sz_bytes(256, 320, 128) == 0
    assert w4.bf16_workspace_bytes(3, 512) == 3 * 512 * 2 + 16
    assert w4.bf16_workspace_bytes(1, 100) == 0


# ---- repacking: C++ vs the independent layout model, and round trips

@pytest.mark.parametrize("group", [64, 32, 128])
@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("N,K", [(16, 64), (16, 128), (32, 192), (48, 512), (16, 320)])
def test_repack_matches_spec(bits, N, K, group):
    if K % max(64, group):
        pytest.skip("groups of 128 need K % 128 == 0")
    rng = np.random.default_rng(N * 1000 + K + bits + group)
    ws = make_weights(rng, "w", N, K, bits, ("real", 0, 1 << bits), (0.001, 0.05), group=group)
    w, s, z = w4.repack(ws.lo, ws.hi, ws.scales, ws.zeros, bits, group)
    w2, s2, z2 = spec_pack(ws.q.astype(np.int64), ws.scales, ws.zeros, bits, group)
    assert np.array_equal(w, w2)
    assert np.array_equal(s, s2)
    assert np.array_equal(z, z2)
    q, su, zu = spec_unpack(w, s, z, N, K, bits, group)
    assert np.array_equal(q, ws.q.astype(np.int64))
    assert np.array_equal(su, ws.scales.view(np.uint16))
    assert np.array_equal(zu, ws.zeros.view(np.uint16))


@pytest.mark.parametrize("bits", [4, 5])
def test_repack_every_code_every_slot(bits):
    """Each code value at each (lane, dword, slot) position survives the round trip."""
    N, K = 16, 128
    nv = 1 << bits
    for shift in range(nv):
        q = ((np.arange(N * K).reshape(N, K) + shift) % nv).astype(np.uint8)
        lo, hi = pack_canonical(q, bits)
        s = np.ones((N, K // 64), dtype=np.float16)
        z = np.zeros((N, K // 64), dtype=np.float16)
        w, sp, zp = w4.repack(lo, hi, s, z, bits)
        qq, _, _ = spec_unpack(w, sp, zp, N, K, bits)
        assert np.array_equal(qq, q.astype(np.int64))


@pytest.mark.parametrize("bits", [4, 5])
def test_repack_pair_interleaves_row_tiles(bits):
    rng = np.random.default_rng(3)
    N, K = 48, 256
    g = make_weights(rng, "g", N, K, bits, ("uniform", 6, 9), (0.005, 0.02))
    u = make_weights(rng, "u", N, K, bits, ("uniform", 6, 9), (0.005, 0.02))
    w, s, z = w4.repack_pair((g.lo, g.hi, g.scales, g.zeros), (u.lo, u.hi, u.scales, u.zeros), bits)
    # expected: packed rows = [g tile 0, u tile 0, g tile 1, u tile 1, ...]
    rows = []
    for i in range(N // 16):
        rows.append(np.arange(16 * i, 16 * i + 16))
    qi = np.concatenate([np.concatenate([g.q[r], u.q[r]]) for r in rows])
    si = np.concatenate([np.concatenate([g.scales[r], u.scales[r]]) for r in rows])
    zi = np.concatenate([np.concatenate([g.zeros[r], u.zeros[r]]) for r in rows])
    w2, s2, z2 = spec_pack(qi.astype(np.int64), si, zi, bits)
    assert np.array_equal(w, w2) and np.array_equal(s, s2) and np.array_equal(z, z2)


def test_repack_concat_is_byte_concat():
    """Packing a row-concatenation equals concatenating the packed parts (shared-X parents)."""
    rng = np.random.default_rng(4)
    a = make_weights(rng, "a", 32, 256, 4, ("uniform", 6, 9), (0.005, 0.02))
    b = make_weights(rng, "b", 48, 256, 4, ("uniform", 6, 9), (0.005, 0.02))
    pa = w4.repack(a.lo, None, a.scales, a.zeros, 4)
    pb = w4.repack(b.lo, None, b.scales, b.zeros, 4)
    pc = w4.repack(np.concatenate([a.lo, b.lo]), None, np.concatenate([a.scales, b.scales]),
                   np.concatenate([a.zeros, b.zeros]), 4)
    for i in range(3):
        assert np.array_equal(pc[i], np.concatenate([pa[i], pb[i]]))


def test_repack_is_deterministic_and_validates():
    rng = np.random.default_rng(8)
    a = make_weights(rng, "a", 32, 256, 5, ("const", 16), (0.0025, 0.01))
    p1 = w4.repack(a.lo, a.hi, a.scales, a.zeros, 5)
    p2 = w4.repack(a.lo, a.hi, a.scales, a.zeros, 5)
    for i in range(3):
        assert np.array_equal(p1[i], p2[i])
    L = w4.lib()
    buf = np.zeros(1 << 16, dtype=np.uint8)
    ptr = buf.ctypes.data_as(ctypes.c_void_p)
    # 5-bit needs the high plane; 4-bit must not get one
    assert L.w4_repack(ptr, None, ptr, ptr, 16, 64, 5, 64, ptr, ptr, ptr) == -1
    assert L.w4_repack(ptr, ptr, ptr, ptr, 16, 64, 4, 64, ptr, ptr, ptr) == -1
    assert L.w4_repack(ptr, None, ptr, ptr, 16, 64, 6, 64, ptr, ptr, ptr) == -2
    assert L.w4_repack(ptr, None, ptr, ptr, 16, 64, 4, 16, ptr, ptr, ptr) == -2
    assert L.w4_repack(ptr, None, ptr, ptr, 16, 64, 4, 128, ptr, ptr, ptr) == -1  # K % 128
    assert L.w4_repack(ptr, None, ptr, ptr, 15, 64, 4, 64, ptr, ptr, ptr) == -1
    assert L.w4_repack(None, None, ptr, ptr, 16, 64, 4, 64, ptr, ptr, ptr) == -1


# ---- grouped call: validation of every matrix and of overlaps between them (fake addresses)

def _grouped(parents, T=4, K=512, x=0x10000, group=64):
    arr = (w4._Parent * max(1, len(parents)))(*[w4._Parent(*p) for p in parents])
    return w4.lib().w4_linear_grouped(x, arr if parents else None, len(parents), T, K, group, None)


def test_grouped_validation():
    a = (0x20000000, 0x30000000, 0x40000000, 256, 4, 0x50000000)
    b = (0x21000000, 0x31000000, 0x41000000, 512, 5, 0x51000000)
    # no GPU here: a valid group passes validation and stops at the device check
    assert _grouped([a, b]) == -6
    assert _grouped([]) == -1                      # no matrix
    assert _grouped([a, b, a[:5] + (0x52000000,), b[:5] + (0x53000000,), a[:5] + (0x54000000,)]) == -1
    assert _grouped([a, b[:4] + (3,) + b[5:]]) == -2                      # 3-bit codes
    assert _grouped([a, b[:3] + (250,) + b[4:]]) == -1                    # N % 16
    assert _grouped([a, b], K=500) == -1                                  # K % 64
    assert _grouped([a, b], group=48) == -2
    assert _grouped([a, b], group=32) == -6
    assert _grouped([a, b[:5] + (0x51000002,)]) == -3                     # misaligned output
    assert _grouped([a, b[:5] + (0x50000000 + 64,)]) == -4                # outputs overlap
    assert _grouped([a, b[:5] + (0x20000000 + 64,)]) == -4                # output over another's codes
    assert _grouped([a, b[:5] + (0x10000 + 16,)]) == -4                   # output over x
    assert _grouped([a, b], T=0) == 0                                     # T == 0: no-op


# ---- bf16 calls: validation of the workspace on top of the fp16 rules (fake addresses)

def _call_bf16(fn, ws=0x70000000, ws_bytes=None, T=4, N=256, K=512, group=64, x=0x10000,
               out=0x50000000):
    L = w4.lib()
    nb = w4.bf16_workspace_bytes(T, K) if ws_bytes is None else ws_bytes
    w, s, z, res = 0x20000000, 0x30000000, 0x40000000, 0x60000000
    if fn == "add":
        return L.w4_linear_add_bf16(x, w, s, z, res, T, N, K, 4, group, out, ws, nb, None)
    if fn == "swiglu":
        return L.w4_linear_swiglu_bf16(x, w, s, z, T, N, K, 4, group, out, ws, nb, None)
    return L.w4_linear_bf16(x, w, s, z, T, N, K, 4, group, out, ws, nb, None)


@pytest.mark.parametrize("fn", ["linear", "swiglu", "add"])
def test_bf16_validation(fn):
    assert _call_bf16(fn) == -6                       # valid: stops at the device check
    assert _call_bf16(fn, group=32) == -6
    assert _call_bf16(fn, ws=0) == -1                 # no workspace
    assert _call_bf16(fn, ws_bytes=100) == -1         # short workspace
    assert _call_bf16(fn, ws=0x70000008) == -3        # misaligned
    assert _call_bf16(fn, ws=0x10000 + 16) == -4      # over x
    assert _call_bf16(fn, ws=0x50000000 - 16) == -4   # over out
    assert _call_bf16(fn, ws=0x30000000) == -4        # over the scales
    assert _call_bf16(fn, T=0, ws=0, x=0, out=0) == 0  # T == 0 is a no-op
    assert _call_bf16(fn, group=16) == -2


def test_noalloc_validation():
    """The allocation-free bf16 call validates like w4_linear_bf16 and rejects, before any
    device work, shapes whose workspace exceeds its static scratch."""
    L = w4.lib()
    args = (0x10000, 0x20000000, 0x30000000, 0x40000000)
    assert L.w4_linear_bf16_noalloc(*args, 4, 256, 512, 4, 64, 0x50000000, None) == -6  # no GPU here
    assert L.w4_linear_bf16_noalloc(*args, 4, 256, 512, 4, 16, 0x50000000, None) == -2
    assert L.w4_linear_bf16_noalloc(*args, 0, 256, 512, 4, 64, 0, None) == 0
    # 4096 x 6144 bf16 activations need 48 MiB of workspace: more than the 32 MiB scratch
    assert w4.bf16_workspace_bytes(4096, 6144) > w4.SCRATCH_BYTES
    assert L.w4_linear_bf16_noalloc(*args, 4096, 5120, 6144, 4, 64, 0x50000000, None) == -8
    assert w4.bf16_workspace_bytes(2048, 6144) <= w4.SCRATCH_BYTES
    assert L.w4_linear_bf16_noalloc(*args, 2048, 5120, 6144, 4, 64, 0x50000000, None) == -6


def test_graph_set_host_side():
    """Graph sets: creation, lookups and misuse are answered on the host (no GPU here)."""
    L = w4.lib()
    g = L.w4_graph_set_create()
    assert g
    assert L.w4_graph_set_has(g, 4) == 0
    assert L.w4_graph_set_launch(g, 4, None) == -5            # nothing recorded for width 4
    assert L.w4_graph_set_begin(g, 4, None) == -1             # the null stream cannot be captured
    assert L.w4_graph_set_begin(None, 4, 0x1234) == -1
    assert L.w4_graph_set_begin(g, -1, 0x1234) == -1
    assert L.w4_graph_set_end(g, 4, 0x1234) == -1             # no capture in progress
    L.w4_graph_set_destroy(g)
    L.w4_graph_set_destroy(None)


def test_a8_validation():
    """A8 calls: workspace size and placement, group 64 only, validation before device work."""
    L = w4.lib()
    T, N, K = 4, 256, 512
    nb = w4.a8_workspace_bytes(T, K)
    assert nb == 4 * 512 + 4 * 4 * 2 * 4 and w4.a8_workspace_bytes(1, 100) == 0
    x, w, s, z, out, ws = 0x10000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, 0x70000000
    assert L.w4_linear_a8(x, w, s, z, T, N, K, 4, 64, out, ws, nb, None) == -6      # valid: no GPU here
    assert L.w4_linear_a8(0, w, s, z, T, N, K, 4, 64, out, ws, nb, None) == -6      # pre-quantised
    assert L.w4_linear_a8(x, w, s, z, T, N, K, 4, 32, out, ws, nb, None) == -2      # group 64 only
    assert L.w4_linear_a8(x, w, s, z, T, N, K, 4, 16, out, ws, nb, None) == -2
    assert L.w4_linear_a8(x, w, s, z, T, N, K, 4, 64, out, ws, nb - 1, None) == -1  # short workspace
    assert L.w4_linear_a8(x, w, s, z, T, N, K, 4, 64, out, 0, nb, None) == -1
    assert L.w4_linear_a8(x, w, s, z, T, N, K, 4, 64, out, ws + 8, nb, None) == -3
    assert L.w4_linear_a8(x, w, s, z, T, N, K, 4, 64, out, out - 64, nb, None) == -4  # over out
    assert L.w4_linear_add_a8(x, w, s, z, 0x60000000, T, N, K, 5, 64, out, 0x60000000 - 16, nb, None) == -4
    assert L.w4_linear_a8(x, w, s, z, 0, N, K, 4, 64, 0, 0, 0, None) == 0           # T == 0
    assert L.w4_quantize_a8(x, T, K, ws, nb, None) == -6
    assert L.w4_quantize_a8(x, T, K, x + 64, nb, None) == -4
    assert L.w4_quantize_a8(x, T, 100, ws, nb, None) == -1
