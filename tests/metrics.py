"""Error metric for parity checks.

Normwise relative error per (batch, head): ||x - ref||_inf / ||ref||_inf over the head's
slice (o: every token and value channel; S: the dk x dv state), and the maximum over heads.
Elementwise relative error is ill-posed where the reference is near zero, so it is not the
gate; the tolerance applies to this normwise figure.
"""
from __future__ import annotations

import numpy as np


def _np(x):
    if hasattr(x, "detach"):
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, np.float64)


def _ratio(num, den):
    # NaN anywhere must fail the check, so it is propagated rather than masked.
    if np.isnan(num).any():
        return float("nan")
    r = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)  # zero reference: absolute
    return float(np.max(r)) if r.size else 0.0


def err_o(o, ref):
    """o, ref: [B, T, H, dv] -> max over (b, h) of the normwise relative error."""
    o, ref = _np(o), _np(ref)
    if o.shape != ref.shape:
        raise ValueError(f"shape {o.shape} vs {ref.shape}")
    if o.size == 0:
        return 0.0
    num = np.abs(o - ref).max(axis=(1, 3))
    den = np.abs(ref).max(axis=(1, 3))
    return _ratio(num, den)


def err_S(S, ref):
    """S, ref: [B, H, dk, dv] -> max over (b, h) of the normwise relative error."""
    S, ref = _np(S), _np(ref)
    if S.shape != ref.shape:
        raise ValueError(f"shape {S.shape} vs {ref.shape}")
    num = np.abs(S - ref).max(axis=(2, 3))
    den = np.abs(ref).max(axis=(2, 3))
    return _ratio(num, den)
