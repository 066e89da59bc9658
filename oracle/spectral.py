"""Token-channel DCT statistics of a gauged KV field -- TEST INFRASTRUCTURE.

"Codec-Gauge: Learning Compression-Friendly Gauges for Transformer KV Caches"
(arXiv HTML), frequency-objective paragraphs: for X' = G X the token axis is
cut into blocks of T_b tokens and a two-dimensional orthonormal DCT is taken
of each T_b x d_l token-channel block (the full head, even when the gauge is
grouped).  With coefficient energy E_uv = U_uv^2 and a normalized radius
r_uv, the frequency term is a spectral centroid; the rate term is a smooth
concave log-amplitude proxy with tau = 0.04; the objective combines them with
lambda_f = 1.0 and lambda_r = 0.02 (gauge-training paragraph).  The
equations themselves are missing from the page; the readings used (DCT-II,
r_uv = sqrt((u/(T_b-1))^2 + (v/(d-1))^2)/sqrt(2), per-block centroid
averaged over blocks, rate = mean log(1 + U^2/tau^2) -- smooth in U and
concave in the energy E = U^2, as the page's energy-preservation argument
needs -- and L = lambda_f L_freq + lambda_r L_rate) are the plainest ones
the surrounding text supports.

Everything is fp64 and written as the plain definition: U = C_Tb X'_blk C_d^T
with explicit DCT matrices, plain sums, and the gradient by the chain rule
(dL/dU -> dL/dX' = C_Tb^T dL/dU C_d -> dL/dG_r = sum_t dL/dx'_t[r] x_t[r]^T
-> dL/dA through the Frechet derivative of exp).
"""
from __future__ import annotations

import numpy as np

from .linalg import gauge_from_skew, grad_A_from_grad_G


def dct_matrix(N: int) -> np.ndarray:
    """Orthonormal DCT-II: C[k, n] = a_k cos(pi (2n+1) k / (2N)),
    a_0 = sqrt(1/N), a_k = sqrt(2/N)."""
    k = np.arange(N)[:, None].astype(np.float64)
    n = np.arange(N)[None, :].astype(np.float64)
    C = np.cos(np.pi * (2.0 * n + 1.0) * k / (2.0 * N))
    C *= np.sqrt(2.0 / N)
    C[0, :] = np.sqrt(1.0 / N)
    return C


def radius_matrix(Tb: int, d: int) -> np.ndarray:
    """r[u, v] = sqrt((u/(Tb-1))^2 + (v/(d-1))^2) / sqrt(2), in [0, 1]."""
    u = np.arange(Tb)[:, None] / (Tb - 1.0)
    v = np.arange(d)[None, :] / (d - 1.0)
    return np.sqrt(u * u + v * v) / np.sqrt(2.0)


def block_diag_gauge(G: np.ndarray) -> np.ndarray:
    """[R, g, g] group gauges -> the full d x d block-diagonal matrix."""
    R, g, _ = G.shape
    full = np.zeros((R * g, R * g))
    for r in range(R):
        full[r * g:(r + 1) * g, r * g:(r + 1) * g] = G[r]
    return full


def dct_stats_field(x: np.ndarray, A: np.ndarray | None, g: int, Tb: int = 16,
                    tau: float = 0.04, lambda_f: float = 1.0,
                    lambda_r: float = 0.02, grad: bool = True,
                    G: np.ndarray | None = None) -> dict:
    """Statistics of one field x [T, d] (raw, un-gauged KV values) under the
    gauge exp(A_r - A_r^T) per group (A [d/g, g, g], fp64).  g = 0 means the
    identity gauge.  An explicit G [d/g, g, g] may be given instead of A (then
    no dA is returned).  Returns a dict with per-field L_freq, L_rate, L,
    sum_E, the per-block centroids, the coefficients U [blocks, Tb, d], and
    (grad=True) dG and dA."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    assert T % Tb == 0
    if g == 0:
        Gfull = np.eye(d)
        Gs = None
    else:
        Gs = gauge_from_skew(A) if G is None else np.asarray(G, np.float64)
        Gfull = block_diag_gauge(Gs)
    xp = x @ Gfull.T                     # x'_t = G x_t for every token
    nb = T // Tb
    blocks = xp.reshape(nb, Tb, d)
    Ct = dct_matrix(Tb)
    Cd = dct_matrix(d)
    U = Ct[None] @ blocks @ Cd.T[None]  # per block: C_Tb X'_blk C_d^T
    E = U * U
    r = radius_matrix(Tb, d)
    SE = E.sum(axis=(1, 2))
    SRE = (r[None] * E).sum(axis=(1, 2))
    Lb = np.where(SE > 0, SRE / np.where(SE > 0, SE, 1.0), 0.0)
    Nc = U.size
    L_freq = Lb.mean()
    L_rate = np.log1p(U * U / (tau * tau)).sum() / Nc
    out = {"L_freq": float(L_freq), "L_rate": float(L_rate),
           "L": float(lambda_f * L_freq + lambda_r * L_rate),
           "sum_E": float(SE.sum()), "L_block": Lb, "U": U}
    if not grad:
        return out
    safe = np.where(SE > 0, SE, 1.0)[:, None, None]
    dU = (lambda_f / nb) * np.where(SE[:, None, None] > 0,
                                    2.0 * U * (r[None] - Lb[:, None, None]) / safe, 0.0)
    dU = dU + (lambda_r / Nc) * 2.0 * U / (tau * tau + U * U)
    dXp = (Ct.T[None] @ dU @ Cd[None]).reshape(T, d)
    if g == 0:
        out["dG"] = None
        out["dA"] = None
        return out
    R = d // g
    dG = np.zeros((R, g, g))
    for rr in range(R):
        sl = slice(rr * g, (rr + 1) * g)
        dG[rr] = dXp[:, sl].T @ x[:, sl]   # sum_t dL/dx'_t[r] x_t[r]^T
    out["dG"] = dG
    out["dA"] = grad_A_from_grad_G(A, dG) if (A is not None and G is None) else None
    return out
