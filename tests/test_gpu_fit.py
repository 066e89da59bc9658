"""GPU checks of gauge training and the coordinate controls ("Codec-Gauge",
arXiv HTML, gauge-training and coordinate-control paragraphs): per-group
second moments and the KLT built from them against the oracle, and a short
AdamW run on the frequency objective that must lower it."""
import numpy as np
import pytest

from fixed_rate_compression_amd import binding as cg
from fixed_rate_compression_amd import fit
from gpu_util import D, kv_cpu, kv_gpu, n_fields, to_dev
from oracle import gaugefit as gf

pytestmark = pytest.mark.gpu


def f64(x):
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if x.dtype == np.uint16 \
        else x.astype(np.float64)


@pytest.mark.parametrize("g,bf16", [(8, True), (16, True), (32, False), (128, True)])
def test_second_moments_and_klt_match_oracle(g, bf16):
    L, KV, B, H, T, cap = 1, 2, 2, 2, 64 * 70 + 16, 64 * 72   # two 4096-row chunks, ragged
    x = kv_cpu(600 + g, L, KV, B, H, T, cap, 0.95, 4, bf16=bf16)
    M = fit.second_moments(to_dev(x), L, KV, B, H, g, tokens=T)
    R = D // g
    for ls in range(L * KV):
        for h in range(H):
            ref = np.zeros((R, g, g))
            for b in range(B):
                f = (ls * B + b) * H + h
                ref += gf.second_moments(f64(x[f, :T]), g)
            got = M[ls // KV, ls % KV, h]
            assert np.max(np.abs(got - ref) / np.max(np.abs(ref))) < 1e-13
            if g <= 32:
                K = fit.control_gauges("klt", 1, 1, 1, g, moments=got[None, None, None])[0, 0, 0]
                for r in range(R):
                    assert np.max(np.abs(K[r] - gf.klt(ref[r]))) < 1e-4


def test_controls_have_block_structure_and_are_orthogonal():
    for kind in ("identity", "hadamard", "dct", "random"):
        G = fit.control_gauges(kind, 2, 2, 3, 16, seed=5)
        assert G.shape == (2, 2, 3, 8, 16, 16)
        Gd = G.reshape(-1, 16, 16).astype(np.float64)
        assert np.max(np.abs(Gd @ Gd.transpose(0, 2, 1) - np.eye(16))) < 1e-5
    r1 = fit.control_gauges("random", 1, 1, 1, 16, seed=1)
    r2 = fit.control_gauges("random", 1, 1, 1, 16, seed=2)
    assert not np.allclose(r1, r2)


def test_training_lowers_the_objective():
    L, KV, B, H, Tw, W = 1, 2, 1, 2, 1024, 4
    x = kv_gpu(610, L, KV, B, H, Tw * W, Tw * W, 0.95, 4, bf16=True)
    held = kv_gpu(611, L, KV, B, H, Tw * 2, Tw * 2, 0.95, 4, bf16=True)
    tr = fit.GaugeTrainer(x, L, KV, B, H, 16, window=Tw, lr=1e-2)
    before = fit.evaluate(held, L, KV, B, H, 16, None, rates=(4,))
    tr.fit(epochs=5)
    assert len(tr.history) == 5 * W
    first = np.mean(tr.history[:W])
    last = np.mean(tr.history[-W:])
    assert last < first, (first, last)
    after = fit.evaluate(held, L, KV, B, H, 16, tr.gauges(), rates=(4,))
    assert after["L"] < before["L"], (before, after)
    assert 0.0 < after["zfp4_nrmse"] < 1.0 and 0.0 < before["zfp4_nrmse"] < 1.0
    # the identity-coordinate evaluation equals an identity control gauge
    ident = fit.evaluate(held, L, KV, B, H, 16, fit.control_gauges("identity", L, KV, H, 16), rates=(4,))
    assert ident["L"] == pytest.approx(before["L"], rel=1e-12)
    assert ident["zfp4_nrmse"] == pytest.approx(before["zfp4_nrmse"], rel=1e-12)


def test_trainer_checkpoint_resume_is_exact(tmp_path):
    # the statistics and the update are deterministic, so training 2 epochs,
    # saving, and resuming in a new trainer for 1 more epoch gives exactly
    # the parameters of 3 uninterrupted epochs
    L, KV, B, H, Tw, W = 1, 2, 1, 2, 512, 3
    x = kv_gpu(620, L, KV, B, H, Tw * W, Tw * W, 0.95, 4, bf16=True)
    ref = fit.GaugeTrainer(x, L, KV, B, H, 16, window=Tw, lr=1e-2)
    ref.fit(epochs=3)
    tr = fit.GaugeTrainer(x, L, KV, B, H, 16, window=Tw, lr=1e-2)
    tr.fit(epochs=2)
    tr.save(tmp_path / "trainer.npz")
    tr2 = fit.GaugeTrainer(x, L, KV, B, H, 16, window=Tw).load(tmp_path / "trainer.npz")
    assert tr2.hyper["lr"] == 1e-2 and tr2.t == 2 * W
    tr2.fit(epochs=1)
    assert np.array_equal(tr2.A, ref.A) and np.array_equal(tr2.m, ref.m) and np.array_equal(tr2.v, ref.v)
    assert tr2.history == ref.history
    other = fit.GaugeTrainer(x, L, KV, B, H, 8, window=Tw)
    with pytest.raises(ValueError):
        other.load(tmp_path / "trainer.npz")
