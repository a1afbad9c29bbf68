"""Helpers shared by the GPU tests: device upload, oracle comparison, tolerance."""
from __future__ import annotations

import numpy as np

import oracle

REL_L2_TOL = 2e-3       # relative L2 error bound against the fp64 oracle
ELEM_TOL = 1e-2         # |y - y_ref| <= ELEM_TOL * (1 + |y_ref|) element-wise


def assert_close(got, ref, what="", elem=True):
    """GPU result vs unrounded fp64 oracle: rel L2 and (unless elem is False, for inputs outside
    the domain where the fp16-weight arithmetic meets it) the per-element bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rel = oracle.rel_l2(got, ref)
    assert rel <= REL_L2_TOL, f"{what}: rel_l2 {rel:.3e} > {REL_L2_TOL}"
    err = float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref)))) if got.size else 0.0
    if elem:
        assert err <= ELEM_TOL, f"{what}: max element error {err:.3e} > {ELEM_TOL}"
    return rel, err


def to_np(t):
    return t.detach().cpu().numpy()


def canon(ws):
    """(lo, hi, scales, zeros) tuple of a synth WeightSet."""
    return (ws.lo, ws.hi, ws.scales, ws.zeros)
