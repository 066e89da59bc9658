"""fp64 matrix exponential and its Frechet derivative -- TEST INFRASTRUCTURE.

The gauge of the Codec-Gauge paper ("Codec-Gauge: Learning Compression-
Friendly Gauges for Transformer KV Caches", arXiv HTML, gauge
parameterization paragraph) is G = exp(A - A^T); the skew-symmetric argument
makes G orthogonal with no penalty term.  Training the gauge with AdamW
(same page, gauge-training paragraph) needs dL/dA, which goes through the
Frechet derivative of exp.

Method (plain and slow on purpose):
  * exp(M): scaling and squaring around a truncated Taylor series,
      exp(M) = (sum_{k<=K} (M/2^s)^k / k!)^(2^s),
    with s chosen so that ||M/2^s||_1 <= 1/4 and terms added until they no
    longer change the sum in fp64.
  * L_exp(M, E) = d/dt exp(M + tE) at t = 0 is the upper-right block of
    exp([[M, E], [0, M]]) (the block-triangular identity of Van Loan 1978;
    Higham, Functions of Matrices, 2008, Thm 3.6), evaluated with the same
    exp.  The gradient of a scalar loss through G = exp(S) is
    dL/dS = L_exp(S^T, dL/dG) (adjoint of the Frechet derivative), and with
    S = A - A^T, dL/dA = dL/dS - (dL/dS)^T.
"""
from __future__ import annotations

import numpy as np


def _onenorm(M: np.ndarray) -> np.ndarray:
    return np.abs(M).sum(axis=-2).max(axis=-1)


def expm(M: np.ndarray) -> np.ndarray:
    """exp of a square matrix or a stack [..., n, n], fp64."""
    M = np.asarray(M, dtype=np.float64)
    n = M.shape[-1]
    flat = M.reshape(-1, n, n)
    out = np.empty_like(flat)
    eye = np.eye(n)
    for b in range(flat.shape[0]):
        A = flat[b]
        nrm = float(_onenorm(A))
        s = 0
        while nrm / (2.0 ** s) > 0.25:
            s += 1
        X = A / (2.0 ** s)
        total = eye.copy()
        term = eye.copy()
        for k in range(1, 60):
            term = term @ X / k
            new_total = total + term
            if np.array_equal(new_total, total):
                break
            total = new_total
        for _ in range(s):
            total = total @ total
        out[b] = total
    return out.reshape(M.shape)


def expm_frechet(M: np.ndarray, E: np.ndarray) -> np.ndarray:
    """Frechet derivative of exp at M in direction E (upper-right block of
    exp([[M, E], [0, M]])).  Works on stacks [..., n, n]."""
    M = np.asarray(M, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    n = M.shape[-1]
    big = np.zeros(M.shape[:-2] + (2 * n, 2 * n))
    big[..., :n, :n] = M
    big[..., :n, n:] = E
    big[..., n:, n:] = M
    return expm(big)[..., :n, n:]


def gauge_from_skew(A: np.ndarray) -> np.ndarray:
    """G = exp(A - A^T) in fp64, for one matrix or a stack."""
    A = np.asarray(A, dtype=np.float64)
    S = A - np.swapaxes(A, -1, -2)
    return expm(S)


def grad_A_from_grad_G(A: np.ndarray, dG: np.ndarray) -> np.ndarray:
    """Chain rule through G = exp(A - A^T): given dL/dG, return dL/dA."""
    A = np.asarray(A, dtype=np.float64)
    S = A - np.swapaxes(A, -1, -2)
    Psi = expm_frechet(np.swapaxes(S, -1, -2), dG)
    return Psi - np.swapaxes(Psi, -1, -2)
