"""Gauge training and coordinate controls -- TEST INFRASTRUCTURE.

"Codec-Gauge: Learning Compression-Friendly Gauges for Transformer KV Caches"
(arXiv HTML):
 - gauge-training paragraph: the gauge parameters are optimized with AdamW
   for 25 epochs over 64 windows of 4096 tokens (hyper-parameters of the
   optimizer are not given; the usual AdamW defaults are used: lr 1e-3,
   betas (0.9, 0.999), eps 1e-8, decoupled weight decay 1e-2);
 - main-grid and coordinate-control paragraphs: identity, random orthogonal
   gauges with the learned gauge's block structure, Hadamard, DCT and PCA/KLT
   controls, the last from the uncentered second-moment eigenbasis at the same
   layer, K/V, head and group granularity.
Plain numpy in fp64, written from the definitions.
"""
from __future__ import annotations

import numpy as np


def adamw_step(p, grad, m, v, t, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=1e-2):
    """One AdamW step (Loshchilov and Hutter, decoupled weight decay), step
    number t >= 1.  Returns new (p, m, v)."""
    p = np.asarray(p, np.float64) * (1.0 - lr * wd)
    m = beta1 * m + (1.0 - beta1) * grad
    v = beta2 * v + (1.0 - beta2) * grad * grad
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    return p - lr * mhat / (np.sqrt(vhat) + eps), m, v


def hadamard(g: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order g (a power of two), scaled by
    1/sqrt(g) so that it is orthogonal."""
    H = np.ones((1, 1))
    while H.shape[0] < g:
        H = np.block([[H, H], [H, -H]])
    assert H.shape[0] == g
    return H / np.sqrt(g)


def dct(g: int) -> np.ndarray:
    """Orthonormal DCT-II matrix C[k, n] = a_k cos(pi (2n + 1) k / (2g))."""
    k = np.arange(g)[:, None]
    n = np.arange(g)[None, :]
    C = np.sqrt(2.0 / g) * np.cos(np.pi * (2 * n + 1) * k / (2 * g))
    C[0] /= np.sqrt(2.0)
    return C


def orthonormalize(M: np.ndarray) -> np.ndarray:
    """Q of the QR factorization of M with R's diagonal made positive: for a
    matrix of independent N(0, 1) entries this is Haar-distributed (Mezzadri
    2007)."""
    Q, R = np.linalg.qr(np.asarray(M, np.float64))
    return Q * np.sign(np.diag(R))[None, :]


def second_moments(x: np.ndarray, g: int) -> np.ndarray:
    """x [T, d] -> [d/g, g, g] uncentered second moments sum_t x_t[r] x_t[r]^T."""
    x = np.asarray(x, np.float64)
    T, d = x.shape
    xr = x.reshape(T, d // g, g)
    return np.einsum("tri,trk->rik", xr, xr)


def klt(M: np.ndarray) -> np.ndarray:
    """Gauge from a symmetric second moment M [g, g]: the rows are the
    eigenvectors in order of decreasing eigenvalue, each with its largest-
    magnitude component (first one on ties) positive.  x' = G x."""
    w, V = np.linalg.eigh(np.asarray(M, np.float64))
    order = np.argsort(-w, kind="stable")
    V = V[:, order]
    for j in range(V.shape[1]):
        i = int(np.argmax(np.abs(V[:, j])))
        if V[i, j] < 0:
            V[:, j] = -V[:, j]
    return V.T
