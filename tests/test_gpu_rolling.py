"""GPU parity of the rolling compressed history ("Codec-Gauge", arXiv HTML,
evaluation-protocol paragraph: each compressed condition keeps its own
history; every new token passes through gauge, backend, decode and inverse
gauge).  After any number of appends the payload must equal a one-shot
encode of the same rows (bit-exact, since 4x4 blocks are independent and sit
at fixed offsets).  Every-token mode: all t rows, a partial last block row
padded by repeating its last token; the history equals their decode.
Completed-rows mode: the rows of completed block rows, followed by the raw
pending rows.  Decoded rows are compared as in the one-shot decoder tests
(gpu_util.check_decoded: bit-exact fmaf chains, or the split-precision bound
for bf16 storage at g = 16 / 32)."""
import numpy as np
import pytest

import oracle
from fixed_rate_compression_amd import binding as cg
from fixed_rate_compression_amd.rolling import RollingHistory
from gpu_util import D, check_decoded, gauge_of_field, gauges_for, kv_cpu, kv_gpu, n_fields, to_dev, to_host

pytestmark = pytest.mark.gpu


def check(rh, raw_host, G, g, R, fields):
    import torch
    torch.cuda.synchronize()
    t = rh.t
    enc = 4 * (t // 4)
    L, KV, B, H = rh.dims
    per = rh.capacity * D * R // 8
    for f in fields:
        xf = raw_host(f)
        Gf = gauge_of_field(G, f, KV, B, H)
        xg = oracle.gauge_forward(oracle.to_f32(xf[:enc]), Gf, g)
        full = np.zeros((rh.capacity, D), np.float32)
        full[:enc] = xg
        p_ref = np.zeros(per, np.uint8)
        oracle.zfp_encode_field(full, R, t0=0, nt=enc, out=p_ref)
        assert np.array_equal(to_host(rh.payload[f * per:(f + 1) * per]), p_ref), (f, t)
        yg = oracle.zfp_decode_field(p_ref, rh.capacity, D, R, 0, enc)[:enc]
        hist = to_host(rh.history[f])
        check_decoded(hist[:enc], yg, Gf, g, (f, t))
        assert np.array_equal(hist[enc:t], xf[enc:t]), (f, t)


def check_every_token(rh, raw_host, G, g, R, fields):
    import torch
    torch.cuda.synchronize()
    t = rh.t
    L, KV, B, H = rh.dims
    per = rh.capacity * D * R // 8
    for f in fields:
        xf = raw_host(f)
        Gf = gauge_of_field(G, f, KV, B, H)
        xg = oracle.gauge_forward(oracle.to_f32(xf[:t]), Gf, g)
        p_ref = oracle.zfp_encode_field(xg, R, t0=0, nt=t, T_payload=rh.capacity)
        assert np.array_equal(to_host(rh.payload[f * per:(f + 1) * per]), p_ref), (f, t)
        yg = oracle.zfp_decode_field(p_ref, rh.capacity, D, R, 0, t)[:t]
        kept = (rh.keep >> ((f // (B * H)) % KV)) & 1     # kind left in gauged coordinates
        check_decoded(to_host(rh.history[f])[:t], yg, Gf, 0 if kept else g, (f, t))


@pytest.mark.parametrize("T0", [64, 66])
def test_rolling_every_token_g16_rate3(T0):
    L, KV, B, H, steps, cap = 1, 2, 2, 2, 11, 80
    g, R = 16, 3
    raw = kv_cpu(46 + T0, L, KV, B, H, T0 + steps, cap, 0.95, 4, bf16=True)
    rawd = to_dev(raw)
    G = gauges_for(47, L, KV, H, g)
    gauge = cg.make_gauge(g, to_dev(np.ascontiguousarray(G)))
    rh = RollingHistory(L, KV, B, H, cap, gauge, R)
    rh.prefill(rawd, T0)
    F = n_fields(L, KV, B, H)
    check_every_token(rh, lambda f: raw[f], G, g, R, range(F))
    for k in range(steps):
        rh.append(rawd[:, T0 + k])
        check_every_token(rh, lambda f: raw[f], G, g, R, range(F))


@pytest.mark.parametrize("keep", [cg.CG_KEEP_VALUES, cg.CG_KEEP_KEYS | cg.CG_KEEP_VALUES])
def test_rolling_every_token_gauged_history(keep):
    # recovery folded into the consumer: the kept kinds stay gauged in the history
    L, KV, B, H, T0, steps, cap = 2, 2, 1, 2, 62, 7, 72
    g, R = 32, 4
    raw = kv_cpu(48 + keep, L, KV, B, H, T0 + steps, cap, 0.95, 4, bf16=True)
    rawd = to_dev(raw)
    G = gauges_for(49, L, KV, H, g)
    gauge = cg.make_gauge(g, to_dev(np.ascontiguousarray(G)))
    rh = RollingHistory(L, KV, B, H, cap, gauge, R, keep=keep)
    rh.prefill(rawd, T0)
    F = n_fields(L, KV, B, H)
    check_every_token(rh, lambda f: raw[f], G, g, R, range(F))
    for k in range(steps):
        rh.append(rawd[:, T0 + k])
        check_every_token(rh, lambda f: raw[f], G, g, R, range(F))


def test_rolling_small_g32_rate4():
    L, KV, B, H, T0, steps, cap = 2, 2, 2, 2, 64, 14, 80
    g, R = 32, 4
    raw = kv_cpu(44, L, KV, B, H, T0 + steps, cap, 0.95, 4, bf16=True)
    rawd = to_dev(raw)
    G = gauges_for(45, L, KV, H, g)
    gauge = cg.make_gauge(g, to_dev(np.ascontiguousarray(G)))
    rh = RollingHistory(L, KV, B, H, cap, gauge, R, every_token=False)
    rh.prefill(rawd, T0)
    F = n_fields(L, KV, B, H)
    check(rh, lambda f: raw[f], G, g, R, range(F))
    for k in range(steps):
        rh.append(rawd[:, T0 + k])
        if k in (2, 3, 9, 13):
            check(rh, lambda f: raw[f], G, g, R, range(F))


@pytest.mark.parametrize("every_token", [False, True])
def test_rolling_decode_config_sampled(every_token):
    """Rolling-history workload: 64 sequences x 28 layers x 4 KV heads x 128,
    history 8192 tokens (bf16), gauge g = 32, 4 b/v; 9 appends (two block
    rows complete, one pending or partial), encoding each completed 4-token
    block (the workload's mode) or every token; sampled fields checked
    against the oracle."""
    import torch
    L, KV, B, H, T0, cap = 28, 2, 64, 4, 8192, 8448
    g, R = 32, 4
    raw = kv_gpu(4, L, KV, B, H, T0 + 16, cap, 0.95, 4, bf16=True)
    G = gauges_for(104, L, KV, H, g)
    gauge = cg.make_gauge(g, to_dev(np.ascontiguousarray(G)))
    rh = RollingHistory(L, KV, B, H, cap, gauge, R, every_token=every_token)
    rh.prefill(raw, T0)
    for k in range(9):
        rh.append(raw[:, T0 + k])
    F = n_fields(L, KV, B, H)
    fields = [0, 1234, F // 2 + 7, F - 1]
    (check_every_token if every_token else check)(rh, lambda f: to_host(raw[f]), G, g, R, fields)
    del rh, raw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("every_token", [False, True])
def test_rolling_checkpoint_resume_is_exact(tmp_path, every_token):
    # save after 6 appends (a pending or partial block row), restore into a
    # new history and continue: payload and history equal an uninterrupted run
    import torch
    L, KV, B, H, T0, steps, cap = 1, 2, 2, 2, 62, 13, 80
    g, R = 16, 3
    raw = kv_cpu(70 + every_token, L, KV, B, H, T0 + steps, cap, 0.95, 4, bf16=True)
    rawd = to_dev(raw)
    G = gauges_for(71, L, KV, H, g)
    gauge = cg.make_gauge(g, to_dev(np.ascontiguousarray(G)))
    ref = RollingHistory(L, KV, B, H, cap, gauge, R, every_token=every_token)
    ref.prefill(rawd, T0)
    for k in range(steps):
        ref.append(rawd[:, T0 + k])
    rh = RollingHistory(L, KV, B, H, cap, gauge, R, every_token=every_token)
    rh.prefill(rawd, T0)
    for k in range(6):
        rh.append(rawd[:, T0 + k])
    rh.save(tmp_path / "hist.npz")
    del rh
    rh2 = RollingHistory.restore(tmp_path / "hist.npz", gauge)
    assert rh2.t == T0 + 6 and rh2.every_token == every_token
    for k in range(6, steps):
        rh2.append(rawd[:, T0 + k])
    torch.cuda.synchronize()
    assert np.array_equal(to_host(rh2.payload), to_host(ref.payload))
    assert np.array_equal(to_host(rh2.history), to_host(ref.history))
