"""Pins of the cache-side error figures (oracle/metrics.py) against closed
forms, and the library's host summary against the oracle's."""
import ctypes

import numpy as np
import pytest

from oracle import metrics


def test_identity_clone_is_zero():
    x = np.random.default_rng(0).standard_normal((64, 128)).astype(np.float32)
    s = metrics.field_error(x, x)
    assert s[0] == 0.0 and s[2] == 0.0 and s[3] == x.size
    assert s[1] == pytest.approx(float(np.sum(x.astype(np.float64) ** 2)), rel=1e-15)


def test_scaled_copy_has_nrmse_of_the_scale():
    # x_hat = (1 + a) x  =>  NRMSE = |a| exactly, MSE = a^2 mean(x^2)
    x = np.random.default_rng(1).standard_normal((3, 64, 128))
    a = 2.0 ** -7
    per = np.array([metrics.field_error((1 + a) * x[f], x[f]) for f in range(3)])
    s = metrics.summary(per, np.array([0, 1, 0]))
    assert s["nrmse"] == pytest.approx(a, rel=1e-12)
    assert s["key_nrmse"] == pytest.approx(a, rel=1e-12)
    assert s["value_nrmse"] == pytest.approx(a, rel=1e-12)
    assert s["mse"] == pytest.approx(a * a * np.mean(x * x), rel=1e-12)
    assert s["max_abs"] == pytest.approx(a * np.max(np.abs(x)), rel=1e-15)


def test_constant_offset_and_separate_kinds():
    # keys exact, values offset by c: key NRMSE 0, MSE = c^2 / 2, max = c
    x = np.ones((2, 8, 4))
    c = 0.25
    per = np.array([metrics.field_error(x[0], x[0]), metrics.field_error(x[1] + c, x[1])])
    s = metrics.summary(per, np.array([0, 1]))
    assert s["key_nrmse"] == 0.0
    assert s["value_nrmse"] == pytest.approx(c, rel=1e-15)     # sqrt(32 c^2 / 32)
    assert s["mse"] == pytest.approx(c * c / 2, rel=1e-15)
    assert s["max_abs"] == c and s["values"] == 64


def test_library_summary_matches_oracle():
    from fixed_rate_compression_amd import binding as cg
    rng = np.random.default_rng(2)
    L, KV, B, H = 2, 2, 3, 2
    F = L * KV * B * H
    per = np.stack([rng.random(F) * 5, rng.random(F) * 100 + 1, rng.random(F), np.full(F, 4096.0)], 1)
    kinds = (np.arange(F) // (B * H)) % KV
    shape = cg.make_shape(L, KV, B, H, 32, 32, 128, cg.CG_DTYPE_BF16)
    got = cg.cg_cache_error_summary(shape, per)
    ref = metrics.summary(per, kinds)
    for k in ref:
        assert got[k] == pytest.approx(ref[k], rel=1e-14), k
