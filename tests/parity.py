"""Comparison helpers for the GPU parity tests (the oracle is the reference).

Tolerances (floating point outputs, per token row):
  bf16 storage: max_t ||dy_t||_inf / ||y_ref_t||_inf <= 2e-2 and mean |dy| <= 1e-3,
                against the oracle in "bf16" storage mode (same rounding points);
  fp32 storage: max_t ||dy_t||_inf / ||y_ref_t||_inf <= 1e-5.
Rows whose reference is exactly zero (every slot dropped) must be exactly zero.
Integer outputs (indices, counts, offsets, row maps) are compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"bf16": dict(row_rel=2e-2, mae=1e-3), "f32": dict(row_rel=1e-5, mae=None)}


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16, torch.float32):
        return t.to(torch.float64).numpy()
    return t.numpy()


def row_errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got - ref)
    ref_inf = np.abs(ref).max(axis=1)
    zero = ref_inf == 0
    rel = np.where(zero, 0.0, d.max(axis=1) / np.where(zero, 1.0, ref_inf))
    return float(rel.max(initial=0.0)), float(d.mean()) if d.size else 0.0, zero


def assert_close_rows(got, ref, storage: str, what: str = "y"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rel, mae, zero = row_errors(got, ref)
    tol = TOL[storage]
    assert rel <= tol["row_rel"], f"{what}: row max-rel {rel:.3g} > {tol['row_rel']}"
    if tol["mae"] is not None:
        assert mae <= tol["mae"], f"{what}: MAE {mae:.3g} > {tol['mae']}"
    if zero.any():
        assert np.all(got[zero] == 0.0), f"{what}: rows with an all-zero reference are not zero"
    return rel, mae


def compare_routing(idx_gpu: np.ndarray, gate_gpu: np.ndarray, ref: dict):
    """Indices bit-exact except on near-tie tokens (counted); gates to 1e-5
    relative wherever the indices agree. Returns the number of flipped tokens."""
    idx_ref = ref["topk_idx"]
    differ = (idx_gpu != idx_ref).any(axis=1)
    flipped = differ & ref["near_tie"]
    bad = differ & ~ref["near_tie"]
    assert not bad.any(), f"{int(bad.sum())} tokens routed differently without a near tie, e.g. {np.nonzero(bad)[0][:5]}"
    same = ~differ
    g_ref = ref["topk_gate"][same]
    assert np.all(np.abs(gate_gpu[same] - g_ref) <= 1e-5 * np.abs(g_ref) + 1e-30), "gates differ by more than 1e-5 relative"
    return int(flipped.sum())
