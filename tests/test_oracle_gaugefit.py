"""Pins of the gauge-training step and the coordinate controls
(oracle/gaugefit.py): AdamW against torch.optim.AdamW (an independent
implementation), Hadamard/DCT/QR/KLT against their defining properties."""
import numpy as np
import pytest

from oracle import gaugefit as gf


def test_adamw_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    p0 = rng.standard_normal(50)
    grads = [rng.standard_normal(50) for _ in range(7)]
    tp = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    opt = torch.optim.AdamW([tp], lr=3e-3, betas=(0.8, 0.99), eps=1e-7, weight_decay=0.05)
    p, m, v = p0.copy(), np.zeros(50), np.zeros(50)
    for t, g in enumerate(grads, 1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = gf.adamw_step(p, g, m, v, t, lr=3e-3, beta1=0.8, beta2=0.99, eps=1e-7, wd=0.05)
    assert np.max(np.abs(p - tp.detach().numpy())) < 1e-14


def test_adamw_first_step_closed_form():
    # step 1 without decay moves every parameter by lr * sign(grad) (up to eps)
    g = np.array([3.0, -0.5, 1e-3])
    p, _, _ = gf.adamw_step(np.zeros(3), g, np.zeros(3), np.zeros(3), 1, lr=0.1, eps=0.0, wd=0.0)
    assert np.allclose(p, -0.1 * np.sign(g), rtol=0, atol=1e-15)


@pytest.mark.parametrize("g", [8, 16, 32, 128])
def test_hadamard_and_dct_are_orthogonal(g):
    H = gf.hadamard(g)
    assert np.max(np.abs(H @ H.T - np.eye(g))) < 1e-13
    assert np.all(np.abs(np.abs(H) - 1 / np.sqrt(g)) < 1e-15)
    C = gf.dct(g)
    assert np.max(np.abs(C @ C.T - np.eye(g))) < 1e-13
    # DCT-II row k is a cosine of k half periods: row 0 constant, row 1 decreasing
    assert np.allclose(C[0], 1 / np.sqrt(g))
    assert np.all(np.diff(C[1]) < 0)


def test_hadamard_order_2_and_4():
    assert np.allclose(gf.hadamard(2) * np.sqrt(2), [[1, 1], [1, -1]])
    assert np.allclose(gf.hadamard(4) * 2, [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])


def test_orthonormalize_is_orthogonal_and_unique():
    rng = np.random.default_rng(1)
    M = rng.standard_normal((16, 16))
    Q = gf.orthonormalize(M)
    assert np.max(np.abs(Q.T @ Q - np.eye(16))) < 1e-13
    # M = Q R with positive diagonal R (upper triangular)
    R = Q.T @ M
    assert np.all(np.diag(R) > 0) and np.max(np.abs(np.tril(R, -1))) < 1e-12


def test_second_moments_and_klt():
    rng = np.random.default_rng(2)
    # data with a known covariance: x = z S^T, S with orthogonal columns of
    # decreasing norm -> eigenvectors = normalized columns
    g = 8
    Q = gf.orthonormalize(rng.standard_normal((g, g)))
    s = np.array([8.0, 6, 5, 4, 3, 2, 1.5, 1])
    z = rng.standard_normal((200000, g))
    x = (z * s) @ Q.T
    M = gf.second_moments(x, g)[0]
    assert np.allclose(M, x.T @ x)
    G = gf.klt(M)
    assert np.max(np.abs(G @ G.T - np.eye(g))) < 1e-12
    # rows match Q's columns up to sign, in order of decreasing variance
    assert np.min(np.abs(np.sum(G * Q.T, axis=1))) > 0.999
    xp = x @ G.T
    var = np.mean(xp * xp, axis=0)
    assert np.all(np.diff(var) < 0)
    # sign rule: largest-magnitude component of each row positive
    assert np.all(G[np.arange(g), np.argmax(np.abs(G), axis=1)] > 0)
