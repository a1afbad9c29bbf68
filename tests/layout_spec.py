"""Independent numpy model of the packed device layout, written from include/w4gemm.h.

Used only by tests: the C++ repacker must produce exactly ``spec_pack``'s bytes, and
``spec_unpack`` must give back the canonical codes, scales and zeros bit for bit.
"""
from __future__ import annotations

import numpy as np

T_OFF = (0, 2, 8, 10)                 # high-plane offset of dword j
R_OFF = (0, 16, 4, 20, 1, 17, 5, 21)  # high-plane position of slot e


def _kmap(kb: int) -> np.ndarray:
    """k[lane, j, e] for k-block kb, straight from the header's formula."""
    lane = np.arange(64)[:, None, None]
    j = np.arange(4)[None, :, None]
    e = np.arange(8)[None, None, :]
    g = lane // 16
    return 128 * kb + 64 * (j >> 1) + 16 * g + 8 * (j & 1) + e


def _lo_bit(e):
    return 4 * (e >> 1) + 16 * (e & 1)


def _sz_entries(KB: int, group: int):
    """(kb, word, half, group index) for every scale / zero entry of a row, from the header:
    group 64: word r, half h -> group 2 kb + h; group 32: word 16 p + r, half h -> group
    4 kb + 2 h + p; group 128: word r, both halves -> group kb.  (Row r is added by the caller.)"""
    out = []
    for kb in range(KB):
        for h in range(2):
            if group == 64:
                out.append((kb, 0, h, 2 * kb + h))
            elif group == 32:
                for p in range(2):
                    out.append((kb, 16 * p, h, 4 * kb + 2 * h + p))
            elif group == 128:
                out.append((kb, 0, h, kb))
            else:
                raise ValueError(group)
    return out


def spec_pack(q: np.ndarray, scales: np.ndarray, zeros: np.ndarray, bits: int, group: int = 64):
    """Raw codes q[N, K] (+ fp16 s, z [N, K/group]) -> (codes bytes, scales u16, zeros u16)."""
    N, K = q.shape
    KB = -(-K // 128)
    G = K // group
    blk = 1280 if bits == 5 else 1024
    qpad = np.zeros((N, KB * 128), dtype=np.int64)
    qpad[:, :K] = q
    out = np.zeros((N // 16, KB, blk), dtype=np.uint8)
    e = np.arange(8)
    for kb in range(KB):
        kidx = _kmap(kb)                                   # [64, 4, 8]
        rows = (np.arange(64) % 16)[:, None, None]
        for rt in range(N // 16):
            c = qpad[16 * rt + rows, kidx]                 # [64, 4, 8]
            words = ((c & 15) << _lo_bit(e)[None, None, :]).sum(axis=2).astype(np.uint32)
            out[rt, kb, :1024] = words.reshape(-1).view(np.uint8)
            if bits == 5:
                hb = (c >> 4) & 1
                pos = np.array(T_OFF)[None, :, None] + np.array(R_OFF)[None, None, :]
                hiw = (hb << pos).sum(axis=(1, 2)).astype(np.uint32)
                out[rt, kb, 1024:] = hiw.view(np.uint8)
    s16 = np.asarray(scales).view(np.uint16)
    z16 = np.asarray(zeros).view(np.uint16)
    W = 32 if group == 32 else 16
    sp = np.zeros((N // 16, KB, W, 2), dtype=np.uint16)
    zp = np.zeros((N // 16, KB, W, 2), dtype=np.uint16)
    for kb, w0, h, grp in _sz_entries(KB, group):
        if grp < G:
            sp[:, kb, w0:w0 + 16, h] = s16[:, grp].reshape(N // 16, 16)
            zp[:, kb, w0:w0 + 16, h] = z16[:, grp].reshape(N // 16, 16)
    return out.reshape(-1), sp.reshape(-1), zp.reshape(-1)


def spec_unpack(w: np.ndarray, sp: np.ndarray, zp: np.ndarray, N: int, K: int, bits: int,
                group: int = 64):
    """Packed bytes -> (q[N, K] int64, scales u16 [N, K/group], zeros u16 [N, K/group])."""
    KB = -(-K // 128)
    G = K // group
    blk = 1280 if bits == 5 else 1024
    wb = np.asarray(w, dtype=np.uint8).reshape(N // 16, KB, blk)
    q = np.zeros((N, KB * 128), dtype=np.int64)
    e = np.arange(8)
    rows = np.arange(64) % 16
    for rt in range(N // 16):
        for kb in range(KB):
            words = wb[rt, kb, :1024].copy().view(np.uint32).reshape(64, 4).astype(np.int64)
            c = (words[:, :, None] >> _lo_bit(e)[None, None, :]) & 15
            if bits == 5:
                hiw = wb[rt, kb, 1024:].copy().view(np.uint32).astype(np.int64)
                pos = np.array(T_OFF)[None, :, None] + np.array(R_OFF)[None, None, :]
                c = c + 16 * ((hiw[:, None, None] >> pos) & 1)
            kidx = _kmap(kb)
            q[16 * rt + rows[:, None, None], kidx] = c
    W = 32 if group == 32 else 16
    sp = np.asarray(sp, dtype=np.uint16).reshape(N // 16, KB, W, 2)
    zp = np.asarray(zp, dtype=np.uint16).reshape(N // 16, KB, W, 2)
    s = np.zeros((N, G), dtype=np.uint16)
    z = np.zeros((N, G), dtype=np.uint16)
    for kb, w0, h, grp in _sz_entries(KB, group):
        sv = sp[:, kb, w0:w0 + 16, h].reshape(N)
        zv = zp[:, kb, w0:w0 + 16, h].reshape(N)
        if grp < G:
            if group == 128 and h == 1:  # the duplicated half must equal the first
                assert np.array_equal(sv, s[:, grp]) and np.array_equal(zv, z[:, grp])
            s[:, grp] = sv
            z[:, grp] = zv
        else:  # padding group must be zero
            assert not sv.any() and not zv.any()
    if K < KB * 128:
        assert not q[:, K:].any()
    return q[:, :K], s, z
