"""Parity metrics and the oracle-vs-HIP comparison helpers used by the GPU
tests and the smoke check.

Error metric (the pages give none; "max relative error" is read per output
row and per state block):

* output row (t, h):  max_j |x - r| / max(max_j |r|, 1e-3 * max_all |r|)
* state (n, h):       max |X - R| / max |R|

and the reported number is the maximum over rows (states).  Tolerances: 1e-4
for fp32 inputs, 2e-2 for bf16 inputs with fp32 state and accumulation.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}

# (label, output error, state error, tolerance) of every parity check in the
# session, printed by the terminal summary hook in conftest.py so that the
# margins appear at the end of the pytest output.
MARGINS: list = []


def record(label: str, err_o: float, err_s: float, tol: float) -> None:
    MARGINS.append((label, float(err_o), float(err_s), float(tol)))


def _np64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def row_rel_err(x, ref) -> float:
    """Max over rows (all axes but the last) of the row-relative error."""
    x, ref = _np64(x), _np64(ref)
    if ref.size == 0:
        return 0.0
    gmax = float(np.max(np.abs(ref)))
    if gmax == 0.0:
        return float(np.max(np.abs(x)))
    rmax = np.max(np.abs(ref), axis=-1)
    den = np.maximum(rmax, 1e-3 * gmax)
    num = np.max(np.abs(x - ref), axis=-1)
    if not np.all(np.isfinite(x)):
        return float("inf")
    return float(np.max(num / den))


def state_rel_err(x, ref) -> float:
    """Max over (n, h) blocks of max|X - R| / max|R| (absolute if R == 0)."""
    x, ref = _np64(x), _np64(ref)
    if ref.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    lead = ref.shape[:-2]
    xr = x.reshape(lead + (-1,))
    rr = ref.reshape(lead + (-1,))
    den = np.max(np.abs(rr), axis=-1)
    num = np.max(np.abs(xr - rr), axis=-1)
    den = np.where(den == 0.0, 1.0, den)
    return float(np.max(num / den))
