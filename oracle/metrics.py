"""Cache-side error figures -- TEST INFRASTRUCTURE.

"Codec-Gauge: Learning Compression-Friendly Gauges for Transformer KV Caches"
(arXiv HTML), evaluation-protocol paragraphs: cache-side metrics are the
compressed bytes, actual bits/value, KV MSE, KV NRMSE, key and value NRMSE and
the maximum absolute error, and the evaluator writes raw sums and counts.  The
formulas are not on the page; the readings used:
  MSE   = sum (x_hat - x)^2 / N
  NRMSE = sqrt(sum (x_hat - x)^2 / sum x^2)   (over all, key or value fields)
  max   = max |x_hat - x|
all over the decoded values as stored, in fp64.
"""
from __future__ import annotations

import numpy as np


def field_error(x_hat: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Raw sums of one field: [sse, ref_ss, max_abs, values] (fp64)."""
    a = np.asarray(x_hat, np.float64).ravel()
    b = np.asarray(x, np.float64).ravel()
    e = a - b
    return np.array([np.sum(e * e), np.sum(b * b), np.max(np.abs(e)) if e.size else 0.0,
                     float(e.size)])


def summary(per_field: np.ndarray, kinds: np.ndarray) -> dict:
    """per_field [F, 4] raw sums, kinds [F] (0 = key, 1 = value) -> figures."""
    p = np.asarray(per_field, np.float64)
    k = np.asarray(kinds)

    def nrmse(rows):
        e, r = p[rows, 0].sum(), p[rows, 1].sum()
        return float(np.sqrt(e / r)) if r > 0 else (float("inf") if e > 0 else 0.0)

    allr = np.ones(len(p), bool)
    n = p[:, 3].sum()
    return {"mse": float(p[:, 0].sum() / n) if n > 0 else 0.0,
            "nrmse": nrmse(allr),
            "key_nrmse": nrmse(k == 0),
            "value_nrmse": nrmse(k == 1) if np.any(k == 1) else 0.0,
            "max_abs": float(p[:, 2].max()) if len(p) else 0.0,
            "values": float(n)}
