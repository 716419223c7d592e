"""Central finite differences -- [AE] "验证方法": the scalar test loss is
L = sum(W * out) with a fixed random W, so the upstream gradient of ``out``
is W, and each analytic input gradient is compared with
(L(x + h e_i) - L(x - h e_i)) / 2h element by element.  Here everything is
float64 with a small step, so agreement is expected to ~1e-7 relative.
"""
from __future__ import annotations

import numpy as np


def numeric_grad(f, x: np.ndarray, h: float = 1e-6) -> np.ndarray:
    """Gradient of the scalar function f at x by central differences."""
    x = np.array(x, dtype=np.float64, copy=True)
    g = np.zeros_like(x)
    flat, gflat = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + h
        fp = f(x)
        flat[i] = old - h
        fm = f(x)
        flat[i] = old
        gflat[i] = (fp - fm) / (2.0 * h)
    return g


def weighted_loss(W: np.ndarray):
    """L(out) = sum(W * out): the template of [AE] "验证方法"."""
    W = np.asarray(W, dtype=np.float64)
    return lambda out: float(np.sum(W * np.asarray(out, dtype=np.float64)))


def max_rel_err(a, b, floor: float = 1e-8) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), floor))) if a.size else 0.0
