"""Tolerance checks shared by the GPU parity tests.

Bars (element by element against the fp64 oracle on identical inputs):
* fp32 inputs: O within 1e-5 relative to max|O_ref|; lse within 1e-5 relative
  (per row, |lse_ref| floored at 1); dQ/dK/dV within 1e-5 relative to the
  reference's max-norm (this last bar is a reading: the fp32 backward bar is not
  stated elsewhere, it takes the forward's).
* bf16 inputs: O within 2e-2 max-abs; dQ/dK/dV within 5e-2 of the reference's
  max-norm; lse within 1e-3 absolute (a bar derived from the arithmetic: scores
  are fp32 sums of exact bf16 products, so lse carries fp32 rounding only).
* A gradient whose exact value is identically zero must come out within 1e-5
  absolute of zero.
"""
from __future__ import annotations

import numpy as np
import torch

ZERO_GRAD_ABS = 1e-5


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def maxabs(x) -> float:
    return float(np.abs(x).max()) if np.size(x) else 0.0


def fwd_errors(O, lse, O_ref, lse_ref):
    O, lse = f64(O), f64(lse)
    assert np.isfinite(O).all() and np.isfinite(lse).all(), "non-finite output"
    eo = maxabs(O - O_ref)
    el = np.abs(lse - lse_ref)
    return eo, el


def check_fwd(dtype: str, O, lse, O_ref, lse_ref, label=""):
    eo, el = fwd_errors(O, lse, O_ref, lse_ref)
    if dtype == "fp32":
        rel_o = eo / max(maxabs(O_ref), 1e-30)
        rel_l = float((el / np.maximum(np.abs(lse_ref), 1.0)).max())
        assert rel_o <= 1e-5, f"{label} fp32 O rel err {rel_o:.3e}"
        assert rel_l <= 1e-5, f"{label} fp32 lse rel err {rel_l:.3e}"
        return rel_o, rel_l
    assert eo <= 2e-2, f"{label} bf16 O max-abs err {eo:.3e}"
    assert float(el.max()) <= 1e-3, f"{label} bf16 lse abs err {float(el.max()):.3e}"
    return eo, float(el.max())


def check_grad(dtype: str, G, G_ref, name: str, label=""):
    G = f64(G)
    assert np.isfinite(G).all(), f"{label} non-finite {name}"
    e = maxabs(G - G_ref)
    ref = maxabs(G_ref)
    if ref == 0.0:
        # exact gradient is identically zero (e.g. N = 1: P = 1 so dS = 0); the
        # relative bar is undefined, so the result must vanish to fp32 rounding
        # of O(1) terms
        assert e <= ZERO_GRAD_ABS, f"{label} {name} should vanish, got {e:.3e}"
        return e
    bar = 1e-5 if dtype == "fp32" else 5e-2
    assert e <= bar * ref, f"{label} {name} err {e:.3e} vs bar {bar * ref:.3e}"
    return e / ref
