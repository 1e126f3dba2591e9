"""Helpers shared by the tests: golden-fixture parsing and error metrics."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Parse a golden text fixture: ``key v1 v2 ...`` lines, '#' comments. Repeated keys are
    returned as a list of arrays in file order."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            arr = np.array([float(x) for x in vals])
            out.setdefault(key, []).append(arr)
    return out


def max_rel_err(x, y, axes=None):
    """Per-slice infinity-norm relative error max|x - y| / max|y|, maximised over the slices
    that ``axes`` (the axes reduced inside one slice) leave; a slice with max|y| = 0 uses the
    absolute error."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if axes is None:
        num = np.max(np.abs(x - y))
        den = np.max(np.abs(y))
        return float(num / den) if den > 0 else float(num)
    num = np.max(np.abs(x - y), axis=axes)
    den = np.max(np.abs(y), axis=axes)
    r = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(np.max(r))


def per_head_rel_err(x, y):
    """Relative error per (batch, head) slice of a [B,T,H,d] tensor, maximised over slices."""
    return max_rel_err(np.moveaxis(np.asarray(x), 2, 1), np.moveaxis(np.asarray(y), 2, 1),
                       axes=(2, 3))


def state_rel_err(x, y):
    """Relative error per (batch, head) slice of a [B,H,dk,dv] state."""
    return max_rel_err(x, y, axes=(2, 3))


def fro_rel_err(x, y):
    """Relative Frobenius error ||x - y||_F / ||y||_F over the whole tensor."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = np.linalg.norm(y.ravel())
    num = np.linalg.norm((x - y).ravel())
    return float(num / den) if den > 0 else float(num)


def elem_rel_err(x, y, floor=1e-3):
    """Worst element-wise relative error |x - y| / |y| over the entries with |y| above
    ``floor`` times max|y| (smaller entries carry no relative precision)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    keep = np.abs(y) > floor * np.max(np.abs(y))
    if not keep.any():
        return 0.0
    return float(np.max(np.abs(x[keep] - y[keep]) / np.abs(y[keep])))
