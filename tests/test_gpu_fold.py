"""GPU parity of the folded recovery ("Codec-Gauge", arXiv HTML,
gauge-parameterization paragraph: recovery folded into the downstream
projections; key side after the positional encoding).

* cg_gauge_heads (the consumer-side gauge on query rows or W_o rows) is
  bit-exact against the oracle's fmaf-chain gauge_heads for every group size.
* cg_decode_gauged writes the kept kinds in gauged coordinates: for zfp those
  rows equal the oracle's decode of the oracle's codes, bit for bit; the
  other kinds equal cg_decode; for the quantizers and the NONE backend the
  kept rows equal cg_decode with the identity gauge on the same payload.
* A decode-attention step on the decoded cache gives the same output both
  ways (explicit recovery, or gauged cache + folded query and W_o).
"""
import numpy as np
import pytest

import oracle
from fixed_rate_compression_amd import binding as cg
from gpu_util import (D, empty_u8, gauge_of_field, gauges_for, kv_cpu, n_fields, to_dev,
                      to_host)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("g", [0, 8, 16, 32, 128])
@pytest.mark.parametrize("bf16", [True, False])
def test_gauge_heads_bit_exact(g, bf16):
    t = __import__("torch")
    L, KV, B, H, q_heads, rows = 2, 2, 1, 2, 8, 130      # 130 rows: three row chunks, ragged
    G = gauges_for(800 + g, L, KV, H, g)
    shape = cg.make_shape(L, KV, B, H, 64, 64, D, cg.CG_DTYPE_BF16)
    gauge = cg.make_gauge(g, to_dev(np.ascontiguousarray(G)) if G is not None else None)
    rng = np.random.default_rng(801 + g)
    x32 = rng.standard_normal((rows, q_heads * D)).astype(np.float32)
    x = oracle.f32_to_bf16(x32) if bf16 else x32
    dt = cg.CG_DTYPE_BF16 if bf16 else cg.CG_DTYPE_F32
    for layer, kind in ((1, 0), (0, 1)):
        xd = to_dev(x)
        yd = t.zeros_like(xd)
        cg.cg_gauge_heads(shape, gauge, layer, kind, q_heads, rows, dt, xd, yd)
        t.cuda.synchronize()
        y = to_host(yd)
        ref = oracle.gauge_heads(oracle.to_f32(x), None if G is None else G[layer, kind], g, q_heads)
        ref = oracle.from_f32(ref, x.dtype)
        assert np.array_equal(y.view(np.uint16 if bf16 else np.uint32),
                              ref.view(np.uint16 if bf16 else np.uint32)), (layer, kind)


def _encode(x, G, g, codec, L, KV, B, H, T, Tcap, bf16):
    t = __import__("torch")
    shape = cg.make_shape(L, KV, B, H, T, Tcap, D, cg.CG_DTYPE_BF16 if bf16 else cg.CG_DTYPE_F32)
    gauge = cg.make_gauge(g, to_dev(np.ascontiguousarray(G)))
    xd = to_dev(x)
    pb, mb, _ = cg.cg_encoded_bytes(shape, codec)
    pay = empty_u8(pb)
    meta = t.zeros(max(mb // 4, 1), dtype=t.float32, device="cuda") if mb else None
    cg.cg_encode(shape, xd, gauge, codec, 0, T, pay, meta)
    return shape, gauge, xd, pay, meta


def _kind(f, KV, B, H):
    return (f // (B * H)) % KV


@pytest.mark.parametrize("keep", [1, 2, 3])
def test_decode_gauged_zfp_against_oracle(keep):
    t = __import__("torch")
    L, KV, B, H, T, Tcap, R, g = 2, 2, 2, 2, 198, 200, 4, 16   # partial last block row
    x = kv_cpu(810 + keep, L, KV, B, H, T, Tcap, 0.95, 4, bf16=True)
    G = gauges_for(811, L, KV, H, g)
    codec = cg.make_codec(cg.CG_BACKEND_ZFP, R)
    shape, gauge, xd, pay, _ = _encode(x, G, g, codec, L, KV, B, H, T, Tcap, True)
    out = t.zeros_like(xd)
    ref = t.zeros_like(xd)
    cg.cg_decode_gauged(shape, pay, None, gauge, codec, 0, T, keep, out)
    cg.cg_decode(shape, pay, None, gauge, codec, 0, T, ref)
    t.cuda.synchronize()
    out, ref, pay = to_host(out), to_host(ref), to_host(pay)
    per = Tcap * D * R // 8
    for f in range(n_fields(L, KV, B, H)):
        if (keep >> _kind(f, KV, B, H)) & 1:
            xg = oracle.gauge_forward(oracle.to_f32(x[f, :T]), gauge_of_field(G, f, KV, B, H), g)
            p_ref = oracle.zfp_encode_field(xg, R, t0=0, nt=T, T_payload=Tcap)
            assert np.array_equal(pay[f * per:(f + 1) * per], p_ref), f
            yg = oracle.zfp_decode_field(p_ref, Tcap, D, R, t0=0, nt=T)[:T]
            assert np.array_equal(out[f, :T], oracle.f32_to_bf16(yg)), f
        else:
            assert np.array_equal(out[f], ref[f]), f
        assert not np.any(out[f, T:])


@pytest.mark.parametrize("backend,bits,blk,res,g", [
    (cg.CG_BACKEND_BLOCK_UNIFORM, 4, 32, 0, 128),
    (cg.CG_BACKEND_KIVI, 4, 32, 128, 16),
    (cg.CG_BACKEND_KIVI, 2, 32, 128, 128),
    (cg.CG_BACKEND_NONE, 0, 0, 0, 32),
    (cg.CG_BACKEND_ZFP, 3, 0, 0, 128),
])
def test_decode_gauged_other_backends(backend, bits, blk, res, g):
    t = __import__("torch")
    L, KV, B, H, T = 2, 2, 1, 2, 64 * 5 + 32 * 3 + 128
    x = kv_cpu(820 + g, L, KV, B, H, T, T, 0.95, 4, bf16=True)
    G = gauges_for(821 + g, L, KV, H, g)
    codec = cg.make_codec(backend, bits, blk, res)
    shape, gauge, xd, pay, meta = _encode(x, G, g, codec, L, KV, B, H, T, T, True)
    ident = cg.make_gauge(0)
    plain = t.zeros_like(xd)
    full = t.zeros_like(xd)
    cg.cg_decode(shape, pay, meta, ident, codec, 0, T, plain)
    cg.cg_decode(shape, pay, meta, gauge, codec, 0, T, full)
    t.cuda.synchronize()
    plain, full = to_host(plain), to_host(full)
    for keep in (1, 2, 3):
        out = t.zeros_like(xd)
        cg.cg_decode_gauged(shape, pay, meta, gauge, codec, 0, T, keep, out)
        t.cuda.synchronize()
        out = to_host(out)
        for f in range(n_fields(L, KV, B, H)):
            want = plain if (keep >> _kind(f, KV, B, H)) & 1 else full
            assert np.array_equal(out[f], want[f]), (keep, f)


def _attention(q, K, V, Wo, H, q_heads):
    ratio = q_heads // H
    o = np.empty(q_heads * D)
    for h in range(q_heads):
        s = K[h // ratio] @ q[h * D:(h + 1) * D] / np.sqrt(D)
        p = np.exp(s - s.max())
        o[h * D:(h + 1) * D] = (p / p.sum()) @ V[h // ratio]
    return Wo @ o


@pytest.mark.parametrize("g,bf16,tol", [(16, False, 1e-5), (128, False, 1e-5), (32, True, 2e-2)])
def test_folded_attention_step(g, bf16, tol):
    """Decode-attention step of layer 1 on the decoded cache: explicit recovery
    (cg_decode) against the gauged cache with the query and W_o gauged by
    cg_gauge_heads.  fp32: both sides differ only by fp32 rounding; bf16: the
    cache is rounded to bf16 in different coordinates."""
    t = __import__("torch")
    L, KV, B, H, T, q_heads, dm = 2, 2, 1, 2, 256, 8, 64
    x = kv_cpu(830 + g, L, KV, B, H, T, T, 0.95, 4, bf16=bf16)
    G = gauges_for(831 + g, L, KV, H, g)
    codec = cg.make_codec(cg.CG_BACKEND_ZFP, 8)
    shape, gauge, xd, pay, _ = _encode(x, G, g, codec, L, KV, B, H, T, T, bf16)
    explicit = t.zeros_like(xd)
    gauged = t.zeros_like(xd)
    cg.cg_decode(shape, pay, None, gauge, codec, 0, T, explicit)
    cg.cg_decode_gauged(shape, pay, None, gauge, codec, 0, T, cg.CG_KEEP_KEYS | cg.CG_KEEP_VALUES,
                        gauged)
    ex = oracle.to_f32(to_host(explicit)).astype(np.float64)
    layer = 1
    kf = [layer * KV * H + s * H for s in (0, 1)]   # first field of (layer, K) and (layer, V); B = 1
    rng = np.random.default_rng(832)
    q = rng.standard_normal((1, q_heads * D))
    # scores of order 1 (the synthetic keys have outlier channels up to ~100x):
    # a bf16 cache rounded in other coordinates then moves each score by about
    # |s| 2^-8, a bounded change of the softmax
    smax = max(np.max(np.abs(ex[kf[0] + h // (q_heads // H)] @ q[0, h * D:(h + 1) * D]))
               for h in range(q_heads)) / np.sqrt(D)
    q = (q * (2.0 / smax)).astype(np.float32)
    Wo = (rng.standard_normal((dm, q_heads * D)) / np.sqrt(q_heads * D)).astype(np.float32)
    qd, Wd = to_dev(q), to_dev(Wo)
    qf, Wf = t.zeros_like(qd), t.zeros_like(Wd)
    cg.cg_gauge_heads(shape, gauge, layer, 0, q_heads, 1, cg.CG_DTYPE_F32, qd, qf)
    cg.cg_gauge_heads(shape, gauge, layer, 1, q_heads, dm, cg.CG_DTYPE_F32, Wd, Wf)
    t.cuda.synchronize()
    ga = oracle.to_f32(to_host(gauged)).astype(np.float64)
    y1 = _attention(q[0].astype(np.float64), ex[kf[0]:kf[0] + H], ex[kf[1]:kf[1] + H],
                    Wo.astype(np.float64), H, q_heads)
    y2 = _attention(to_host(qf)[0].astype(np.float64), ga[kf[0]:kf[0] + H], ga[kf[1]:kf[1] + H],
                    to_host(Wf).astype(np.float64), H, q_heads)
    err = np.max(np.abs(y1 - y2)) / np.max(np.abs(y1))
    assert err <= tol, err
