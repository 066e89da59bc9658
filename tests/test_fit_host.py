"""The library's host-side gauge-training pieces against the oracle: AdamW
update, control gauges (identity, Hadamard, DCT, Haar QR, KLT)."""
import numpy as np
import pytest

from fixed_rate_compression_amd import binding as cg
from oracle import gaugefit as gf


def test_adamw_update_matches_oracle():
    rng = np.random.default_rng(3)
    n = 1000
    p = rng.standard_normal(n)
    m = np.zeros(n)
    v = np.zeros(n)
    po, mo, vo = p.copy(), m.copy(), v.copy()
    for t in range(1, 6):
        g = rng.standard_normal(n)
        cg.cg_adamw_update(p, g, m, v, t, lr=2e-3, beta1=0.85, beta2=0.995, eps=1e-9, weight_decay=0.03)
        po, mo, vo = gf.adamw_step(po, g, mo, vo, t, lr=2e-3, beta1=0.85, beta2=0.995, eps=1e-9, wd=0.03)
    assert np.max(np.abs(p - po)) < 1e-15
    assert np.max(np.abs(m - mo)) < 1e-15 and np.max(np.abs(v - vo)) < 1e-15


@pytest.mark.parametrize("g", [8, 16, 32, 128])
def test_fixed_controls_match_oracle(g):
    I = cg.cg_gauge_control(cg.CG_CONTROL_IDENTITY, 2, g)
    assert np.array_equal(I[1], np.eye(g, dtype=np.float32))
    H = cg.cg_gauge_control(cg.CG_CONTROL_HADAMARD, 1, g)[0]
    assert np.array_equal(H, gf.hadamard(g).astype(np.float32))
    C = cg.cg_gauge_control(cg.CG_CONTROL_DCT, 1, g)[0]
    assert np.max(np.abs(C - gf.dct(g))) <= 2.0 ** -24


@pytest.mark.parametrize("g", [8, 16, 32, 128])
def test_random_orthogonal_and_klt_match_oracle(g):
    rng = np.random.default_rng(g)
    M = rng.standard_normal((3, g, g))
    Q = cg.cg_gauge_control(cg.CG_CONTROL_ORTHONORMALIZE, 3, g, M)
    for b in range(3):
        assert np.max(np.abs(Q[b] - gf.orthonormalize(M[b]))) < 1e-6
    # second moments with well-separated eigenvalues
    S = np.empty((3, g, g))
    for b in range(3):
        U = gf.orthonormalize(rng.standard_normal((g, g)))
        S[b] = U @ np.diag(np.linspace(10.0, 1.0, g)) @ U.T
    K = cg.cg_gauge_control(cg.CG_CONTROL_KLT, 3, g, S)
    for b in range(3):
        ref = gf.klt(S[b])
        assert np.max(np.abs(K[b] - ref)) < 1e-6
        assert np.max(np.abs(K[b].astype(np.float64) @ K[b].T - np.eye(g))) < 1e-5


def test_control_errors():
    with pytest.raises(cg.CodecGaugeError):
        cg.cg_gauge_control(cg.CG_CONTROL_HADAMARD, 1, 12)
    with pytest.raises(cg.CodecGaugeError):
        cg.cg_gauge_control(cg.CG_CONTROL_KLT, 1, 8, None)
    with pytest.raises(cg.CodecGaugeError):
        cg.cg_gauge_control(9, 1, 8)


@pytest.mark.parametrize("g,scale", [(8, 0.1), (16, 0.1), (32, 0.05), (16, 2.0)])
def test_gauge_grad_matches_oracle_frechet(g, scale):
    # dL/dA through exp: the library's one-pass Pade Frechet derivative against
    # the oracle's block-matrix exponential (Taylor, independent), including a
    # large-norm case that needs scaling and squaring
    from oracle import linalg
    rng = np.random.default_rng(g)
    A = rng.standard_normal((4, g, g)) * scale
    dG = rng.standard_normal((4, g, g))
    got = cg.cg_gauge_grad(A, dG)
    for b in range(4):
        ref = linalg.grad_A_from_grad_G(A[b], dG[b])
        assert np.max(np.abs(got[b] - ref)) <= 1e-11 * max(1.0, np.max(np.abs(ref)))


def test_gauge_file_round_trip_and_check(tmp_path):
    from fixed_rate_compression_amd import fit
    rng = np.random.default_rng(3)
    A = 0.1 * rng.standard_normal((2, 2, 3, 8, 16, 16))
    fit.save_gauges(tmp_path / "g.npz", A, 16)
    A2, G2, g = fit.load_gauges(tmp_path / "g.npz")
    assert g == 16 and np.array_equal(A2, A) and G2.dtype == np.float32
    assert np.array_equal(G2.reshape(-1, 16, 16), cg.cg_gauge_from_skew(A.reshape(-1, 16, 16)))
    # a G that is not exp(A - A^T) of the stored A is refused
    G2.reshape(-1)[5] += 1e-3
    np.savez(tmp_path / "bad.npz", A=A, G=G2, g=np.int32(16))
    with pytest.raises(ValueError):
        fit.load_gauges(tmp_path / "bad.npz")
