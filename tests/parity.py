"""Parity metrics and tolerances shared by the CPU and GPU tests.

Floating-point bar for y (per matrix, over all R x N outputs):
  max_rel = max |y - y_ref| / max |y_ref|   <= 2e-3
  rel_l2  = ||y - y_ref||_2 / ||y_ref||_2   <= 1e-4
The dequantised fp32 weights must match the oracle's single rounding bit for bit.
"""
from __future__ import annotations

import numpy as np

MAX_REL = 2e-3
REL_L2 = 1e-4


def metrics(y: np.ndarray, ref: np.ndarray) -> dict:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    diff = y - ref
    scale = np.abs(ref).max()
    l2 = np.linalg.norm(ref)
    return {
        "max_rel": float(np.abs(diff).max() / scale) if scale > 0 else float(np.abs(diff).max()),
        "rel_l2": float(np.linalg.norm(diff) / l2) if l2 > 0 else float(np.linalg.norm(diff)),
        "max_abs": float(np.abs(diff).max()),
        "finite": bool(np.isfinite(y).all()),
    }


def assert_parity(y, ref, what: str = "") -> dict:
    m = metrics(y, ref)
    assert m["finite"], f"{what}: non-finite output"
    assert m["max_rel"] <= MAX_REL, f"{what}: max_rel {m['max_rel']:.3e} > {MAX_REL}"
    assert m["rel_l2"] <= REL_L2, f"{what}: rel_l2 {m['rel_l2']:.3e} > {REL_L2}"
    return m
