"""Pins of the oracle's fp64 matrix exponential and Frechet derivative.

The gauge is G = exp(A - A^T) ("Codec-Gauge", arXiv HTML, gauge
parameterization paragraph): orthogonal by construction.  The oracle's
Taylor scaling-and-squaring exp is checked against closed forms, group
identities and scipy's independent Pade-based implementation.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import linalg


def test_exp_zero_is_identity_exactly():
    for n in (2, 16, 32):
        assert np.array_equal(linalg.expm(np.zeros((n, n))), np.eye(n))


@pytest.mark.parametrize("a", [0.0, 0.3, -1.2, 2.5, 7.0])
def test_exp_plane_rotation_closed_form(a):
    # S = [[0, a], [-a, 0]]  =>  exp(S) = [[cos a, sin a], [-sin a, cos a]]
    S = np.array([[0.0, a], [-a, 0.0]])
    want = np.array([[np.cos(a), np.sin(a)], [-np.sin(a), np.cos(a)]])
    assert np.max(np.abs(linalg.expm(S) - want)) < 1e-14


def test_gauge_from_skew_g2_closed_form():
    A = np.array([[0.4, 1.1], [0.2, -0.7]])
    a = A[0, 1] - A[1, 0]
    G = oracle.gauge_from_skew(A)
    want = np.array([[np.cos(a), np.sin(a)], [-np.sin(a), np.cos(a)]])
    assert np.max(np.abs(G - want)) < 1e-14


def test_exp_symmetric_by_eigendecomposition():
    rng = np.random.default_rng(3)
    B = rng.standard_normal((12, 12))
    M = 0.3 * (B + B.T)
    w, Q = np.linalg.eigh(M)
    want = (Q * np.exp(w)) @ Q.T
    got = linalg.expm(M)
    assert np.max(np.abs(got - want)) < 1e-12 * np.max(np.abs(want))


def test_exp_nilpotent_closed_form():
    # strictly upper-triangular N with N^3 = 0: exp(N) = I + N + N^2/2
    N = np.array([[0.0, 2.0, -3.0], [0.0, 0.0, 5.0], [0.0, 0.0, 0.0]])
    want = np.eye(3) + N + N @ N / 2.0
    assert np.max(np.abs(linalg.expm(N) - want)) < 1e-14


@pytest.mark.parametrize("g", [4, 16, 32, 128])
def test_exp_matches_scipy_and_is_orthogonal(g):
    rng = np.random.default_rng(g)
    A = 0.1 * rng.standard_normal((3, g, g))
    G = oracle.gauge_from_skew(A)
    for b in range(3):
        S = A[b] - A[b].T
        ref = scipy.linalg.expm(S)
        assert np.max(np.abs(G[b] - ref)) < 1e-12
        assert np.max(np.abs(G[b].T @ G[b] - np.eye(g))) < 1e-13
        # exp(S) exp(-S) = I and exp(S)^T = exp(-S)
        assert np.max(np.abs(G[b] @ linalg.expm(-S) - np.eye(g))) < 1e-13
        assert abs(np.linalg.det(G[b]) - 1.0) < 1e-12


def test_exp_large_norm_scaling_path():
    rng = np.random.default_rng(9)
    A = 3.0 * rng.standard_normal((16, 16))
    S = A - A.T
    assert np.max(np.abs(linalg.expm(S) - scipy.linalg.expm(S))) < 1e-11


def test_frechet_matches_scipy():
    rng = np.random.default_rng(5)
    for n in (3, 8, 16):
        M = 0.2 * rng.standard_normal((n, n))
        E = rng.standard_normal((n, n))
        ref = scipy.linalg.expm_frechet(M, E, compute_expm=False)
        got = linalg.expm_frechet(M, E)
        assert np.max(np.abs(got - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_frechet_commuting_direction_closed_form():
    # for E = M (commutes with M): L(M, M) = M exp(M)
    rng = np.random.default_rng(6)
    M = 0.3 * rng.standard_normal((6, 6))
    want = M @ scipy.linalg.expm(M)
    assert np.max(np.abs(linalg.expm_frechet(M, M) - want)) < 1e-13


def test_grad_A_finite_differences():
    # scalar f(A) = <W, exp(A - A^T)>; df/dA from the oracle vs central FD
    rng = np.random.default_rng(8)
    g = 4
    A = 0.2 * rng.standard_normal((g, g))
    W = rng.standard_normal((g, g))
    dA = linalg.grad_A_from_grad_G(A, W)
    h = 1e-6
    fd = np.zeros_like(A)
    for i in range(g):
        for j in range(g):
            Ap = A.copy(); Ap[i, j] += h
            Am = A.copy(); Am[i, j] -= h
            fd[i, j] = (np.sum(W * oracle.gauge_from_skew(Ap)) -
                        np.sum(W * oracle.gauge_from_skew(Am))) / (2 * h)
    assert np.max(np.abs(dA - fd)) < 1e-8
    assert np.max(np.abs(dA + dA.T)) < 1e-14   # antisymmetric
