"""GPU parity of the fused gauge + zfp-style encode and decode + inverse gauge
against the oracle ("Codec-Gauge", arXiv HTML, evaluation-protocol
paragraph: gauge -> fixed-rate zfp on the FP32-transformed field -> decode ->
inverse gauge).  Bar: bit-exact codec streams.  The decoded cache is
bit-exact wherever the decoder evaluates the inverse gauge as the oracle's
fmaf chains (fp32 storage at every group size; bf16 storage at g = 0 and 8),
because both sides decode the same integers, chain the same fmafs and round
the same way.  With bf16 storage at g = 16 / 32 the inverse gauge runs as
split-precision bf16 matrix-core products: every element is held to the
error bound of that arithmetic (gpu_util.check_decoded) and the 1e-2 bf16
bar.  The full-head gauge with bf16 storage is checked staged."""
import numpy as np
import pytest

import oracle
from fixed_rate_compression_amd import binding as cg
from gpu_util import (D, check_decoded, check_dense_forward, empty_u8, gauge_of_field, gauges_for, kv_cpu, kv_gpu,
                      n_fields, to_dev, to_host, zfp_oracle_decoded)

pytestmark = pytest.mark.gpu


def rel_err(got, ref):
    return float(np.max(np.abs(got.astype(np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))


def run_zfp(x_host, G, g, R, L, KV, B, H, T, Tcap, bf16, chunks=None):
    import torch
    shape = cg.make_shape(L, KV, B, H, T, Tcap, D, cg.CG_DTYPE_BF16 if bf16 else cg.CG_DTYPE_F32)
    codec = cg.make_codec(cg.CG_BACKEND_ZFP, R)
    Gd = to_dev(np.ascontiguousarray(G)) if G is not None else None
    gauge = cg.make_gauge(g, Gd)
    xd = to_dev(x_host)
    nbytes, _ = cg.cg_encoded_bytes(shape, codec)[:2]
    assert nbytes == n_fields(L, KV, B, H) * Tcap * D * R // 8
    pay = empty_u8(nbytes)
    out = torch.zeros_like(xd)
    if chunks is None:
        cg.cg_roundtrip(shape, xd, gauge, codec, pay, None, out)
    else:
        t0 = 0
        for n in chunks:
            cg.cg_encode(shape, xd, gauge, codec, t0, n, pay)
            t0 += n
        assert t0 == T
        cg.cg_decode(shape, pay, None, gauge, codec, 0, T, out)
    torch.cuda.synchronize()
    return to_host(pay), to_host(out)


def check_against_oracle(x, G, g, R, L, KV, B, H, T, Tcap, pay, out, fields=None):
    F = n_fields(L, KV, B, H)
    per = Tcap * D * R // 8
    for f in (range(F) if fields is None else fields):
        Gf = gauge_of_field(G, f, KV, B, H)
        p_ref, yg = zfp_oracle_decoded(x[f], Gf, g, R, T, Tcap)
        assert np.array_equal(pay[f * per:(f + 1) * per], p_ref), f"payload mismatch in field {f}"
        check_decoded(out[f, :T], yg, Gf, g, f"decoded rows of field {f}")


def test_small_config_fp32_g16_rate4():
    # 1 layer x K/V x 2 heads x T=4096, fp32, rho 0.9, 2 outliers, g = 16, 4 b/v
    L, KV, B, H, T = 1, 2, 1, 2, 4096
    x = kv_cpu(1, L, KV, B, H, T, T, 0.9, 2, bf16=False)
    G = gauges_for(101, L, KV, H, 16)
    pay, out = run_zfp(x, G, 16, 4, L, KV, B, H, T, T, False)
    assert pay.size == 4 * T * D * 4 // 8 == 1048576
    check_against_oracle(x, G, 16, 4, L, KV, B, H, T, T, pay, out)


@pytest.mark.parametrize("R", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("g", [0, 8, 16, 32])
def test_bf16_rates_groups_ragged(R, g):
    # T = 200: three full 64-token tiles and a ragged 8-token tile; capacity 256
    L, KV, B, H, T, Tcap = 2, 2, 1, 2, 200, 256
    x = kv_cpu(7 + R, L, KV, B, H, T, Tcap, 0.95, 4, bf16=True)
    G = gauges_for(200 + g, L, KV, H, g)
    pay, out = run_zfp(x, G, g, R, L, KV, B, H, T, Tcap, True)
    check_against_oracle(x, G, g, R, L, KV, B, H, T, Tcap, pay, out)


@pytest.mark.parametrize("g", [0, 8, 32])
def test_fp32_other_groups_batch(g):
    L, KV, B, H, T = 1, 2, 3, 1, 132
    x = kv_cpu(5, L, KV, B, H, T, T, 0.9, 2, bf16=False)
    G = gauges_for(300 + g, L, KV, H, g)
    pay, out = run_zfp(x, G, g, 3, L, KV, B, H, T, T, False)
    check_against_oracle(x, G, g, 3, L, KV, B, H, T, T, pay, out)


@pytest.mark.parametrize("T,g,bf16", [(201, 16, True), (130, 0, False), (67, 32, True), (1, 8, True)])
def test_partial_last_block_row(T, g, bf16):
    # token counts that are not multiples of 4: the last block row is padded
    # by repeating the last token; codes and decoded rows bit-exact
    L, KV, B, H, Tcap = 1, 2, 1, 2, 256
    x = kv_cpu(60 + T, L, KV, B, H, T, Tcap, 0.95, 4, bf16=bf16)
    G = gauges_for(61, L, KV, H, g)
    for R in (3, 4):
        pay, out = run_zfp(x, G, g, R, L, KV, B, H, T, Tcap, bf16)
        check_against_oracle(x, G, g, R, L, KV, B, H, T, Tcap, pay, out)
        assert not np.any(out[:, T:])          # rows past the valid tokens untouched


def test_partial_rows_dense_gauge():
    # full-head gauge with a partial last block row: staged like the other
    # dense-gauge test (gauged values from cg_gauge_apply, codes bit-exact)
    t = __import__("torch")
    L, KV, B, H, T = 1, 1, 1, 2, 64 * 17 + 6
    x = kv_cpu(62, L, KV, B, H, T, T + 2, 0.95, 4, bf16=True)
    G = gauges_for(63, L, KV, H, 128)
    pay, out = run_zfp(x, G, 128, 4, L, KV, B, H, T, T + 2, True)
    shape = cg.make_shape(L, KV, B, H, T, T + 2, D, cg.CG_DTYPE_BF16)
    gauge = cg.make_gauge(128, to_dev(np.ascontiguousarray(G)))
    xg_d = t.zeros((2, T + 2, D), dtype=t.float32, device="cuda")
    cg.cg_gauge_apply(shape, to_dev(x), gauge, 0, xg_d)
    t.cuda.synchronize()
    xg = to_host(xg_d)
    per = (T + 2) * D * 4 // 8
    for f in range(2):
        p_ref = oracle.zfp_encode_field(xg[f, :T], 4, t0=0, nt=T, T_payload=T + 2)
        assert np.array_equal(pay[f * per:(f + 1) * per], p_ref), f


def test_appends_equal_one_shot():
    L, KV, B, H, T, Tcap = 1, 2, 1, 2, 200, 256
    x = kv_cpu(9, L, KV, B, H, T, Tcap, 0.95, 4, bf16=True)
    G = gauges_for(9, L, KV, H, 16)
    one, out1 = run_zfp(x, G, 16, 4, L, KV, B, H, T, Tcap, True)
    inc, out2 = run_zfp(x, G, 16, 4, L, KV, B, H, T, Tcap, True, chunks=[4, 64, 68, 4, 60])
    assert np.array_equal(one, inc)
    assert np.array_equal(out1, out2)


def test_edge_values_zero_constant_denormal_outlier():
    import torch
    L, KV, B, H, T = 1, 1, 1, 1, 64
    x = kv_cpu(3, L, KV, B, H, T, T, 0.9, 2, bf16=False)
    x[0, 0:4, 0:4] = 0.0
    x[0, 0:4, 4:8] = -0.0
    x[0, 4:8, 0:4] = 3.25
    x[0, 8:12, 0:8] = 1e-41           # subnormal
    x[0, 12:16, 0:4] = 3.0e38
    x[0, 16:20, 8:12] = np.array([1e-30, -5e20, 7.0, 0.0] * 4).reshape(4, 4)
    for g in (0, 16):
        G = gauges_for(4, L, KV, H, g)
        for R in (2, 4, 8):
            pay, out = run_zfp(x, G, g, R, L, KV, B, H, T, T, False)
            check_against_oracle(x, G, g, R, L, KV, B, H, T, T, pay, out)


@pytest.mark.parametrize("R", [2, 3, 4, 6, 8])
def test_mixed_value_fields(R):
    """Whole fields of mixed magnitudes through the fused kernels, bit-exact
    streams and decoded rows against the oracle: Gaussian values under
    lognormal channel scales with 10 % zeros, a band of subnormal-scale rows
    and a band of rows near 1e37 (below fp32 overflow after any orthogonal
    16-channel mix), fp32 storage at g = 0 and 16."""
    L, KV, B, H, T = 1, 1, 1, 2, 512
    rng = np.random.default_rng(1100 + R)
    x = rng.standard_normal((2, T, D)) * np.exp(3 * rng.standard_normal((2, 1, D)))
    x[rng.random((2, T, D)) < 0.1] = 0.0
    x[:, 32:64] *= 1e-41
    x[:, 96:128] = x[:, 96:128] / np.max(np.abs(x[:, 96:128])) * 1e37
    x = x.astype(np.float32)
    for g in (0, 16):
        G = gauges_for(1200 + R, L, KV, H, g)
        pay, out = run_zfp(x, G, g, R, L, KV, B, H, T, T, False)
        check_against_oracle(x, G, g, R, L, KV, B, H, T, T, pay, out)


def test_random_payload_decodes_like_oracle():
    """Arbitrary streams (every 16R-bit pattern is a valid fixed-rate block)
    decode exactly like the oracle: uniform random bytes, and bits that are
    mostly 0 (long runs of failed tests and many planes, the 32-plane path)
    or mostly 1 (early caps at coefficient 15, all 16 coefficients
    significant), 32768 blocks per rate and pattern."""
    import torch
    L, KV, B, H, T = 1, 1, 1, 2, 2048
    rng = np.random.default_rng(0)
    for R in (2, 3, 4, 6, 8):
        shape = cg.make_shape(L, KV, B, H, T, T, D, cg.CG_DTYPE_F32)
        codec = cg.make_codec(cg.CG_BACKEND_ZFP, R)
        nbytes = 2 * T * D * R // 8
        for p_one in (0.5, 0.15, 0.85):
            raw = np.packbits(rng.random(8 * nbytes) < p_one, bitorder="little")
            pay = torch.from_numpy(raw).cuda()
            out = torch.zeros((2, T, D), dtype=torch.float32, device="cuda")
            cg.cg_decode(shape, pay, None, cg.make_gauge(0), codec, 0, T, out)
            torch.cuda.synchronize()
            got = to_host(out)
            per = T * D * R // 8
            for f in range(2):
                ref = oracle.zfp_decode_field(raw[f * per:(f + 1) * per], T, D, R)
                assert np.array_equal(got[f].view(np.uint32), ref.view(np.uint32)), (R, p_one, f)


def test_gauge_apply_and_none_backend_bit_exact():
    import torch
    L, KV, B, H, T = 2, 2, 1, 2, 100
    for g in (16, 32):
        x = kv_cpu(11, L, KV, B, H, T, T, 0.95, 4, bf16=True)
        G = gauges_for(12, L, KV, H, g)
        shape = cg.make_shape(L, KV, B, H, T, T, D, cg.CG_DTYPE_BF16)
        gauge = cg.make_gauge(g, to_dev(G))
        xd = to_dev(x)
        out = torch.zeros((n_fields(L, KV, B, H), T, D), dtype=torch.float32, device="cuda")
        cg.cg_gauge_apply(shape, xd, gauge, 0, out)
        codec = cg.make_codec(cg.CG_BACKEND_NONE)
        pay = empty_u8(cg.cg_encoded_bytes(shape, codec)[0])
        back = torch.zeros_like(xd)
        cg.cg_roundtrip(shape, xd, gauge, codec, pay, None, back)
        torch.cuda.synchronize()
        got = to_host(out)
        payf = to_host(pay).view(np.float32).reshape(-1, T, D)
        bk = to_host(back)
        for f in range(n_fields(L, KV, B, H)):
            Gf = gauge_of_field(G, f, KV, B, H)
            ref = oracle.gauge_forward(oracle.to_f32(x[f]), Gf, g)
            assert np.array_equal(got[f].view(np.uint32), ref.view(np.uint32))
            assert np.array_equal(payf[f].view(np.uint32), ref.view(np.uint32))
            inv = oracle.f32_to_bf16(oracle.gauge_inverse(ref, Gf, g))
            assert np.array_equal(bk[f], inv)


def test_identity_clone_is_exact():
    import torch
    L, KV, B, H, T = 1, 2, 1, 2, 64
    for bf16 in (True, False):
        x = kv_cpu(13, L, KV, B, H, T, T, 0.9, 2, bf16=bf16)
        shape = cg.make_shape(L, KV, B, H, T, T, D, cg.CG_DTYPE_BF16 if bf16 else cg.CG_DTYPE_F32)
        codec = cg.make_codec(cg.CG_BACKEND_NONE)
        pay = empty_u8(cg.cg_encoded_bytes(shape, codec)[0])
        xd = to_dev(x)
        back = torch.zeros_like(xd)
        cg.cg_roundtrip(shape, xd, cg.make_gauge(0), codec, pay, None, back)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(back).view(np.uint8), x.view(np.uint8))


def test_llama8b_class_full_size_sampled_fields():
    """The benchmark's workload and launch configuration: 32 layers x K/V x 8
    KV heads x 32768 tokens, bf16, g = 16, 4 b/v; generated on the device.
    Sampled fields (layers 0, 15, 31; both K and V; heads 0 and 7) are
    compared bit-exactly with the oracle; bytes = 4 x values / 8 exactly."""
    import torch
    L, KV, B, H, T = 32, 2, 1, 8, 32768
    R, g = 4, 16
    x = kv_gpu(2, L, KV, B, H, T, T, 0.95, 4, bf16=True)
    G = gauges_for(102, L, KV, H, g)
    shape = cg.make_shape(L, KV, B, H, T, T, D, cg.CG_DTYPE_BF16)
    codec = cg.make_codec(cg.CG_BACKEND_ZFP, R)
    nbytes = cg.cg_encoded_bytes(shape, codec)[0]
    assert nbytes == L * KV * H * T * D * R // 8
    pay = empty_u8(nbytes)
    out = torch.empty_like(x)
    gauge = cg.make_gauge(g, to_dev(G))
    cg.cg_encode(shape, x, gauge, codec, 0, T, pay)
    cg.cg_decode(shape, pay, None, gauge, codec, 0, T, out)
    torch.cuda.synchronize()
    per = T * D * R // 8
    fields = []
    for l in (0, 15, 31):
        for s in (0, 1):
            for h in (0, 7):
                fields.append((l * KV + s) * H + h)
    for f in fields:
        xf = to_host(x[f])
        Gf = gauge_of_field(G, f, KV, B, H)
        p_ref, yg = zfp_oracle_decoded(xf, Gf, g, R, T, T)
        assert np.array_equal(to_host(pay[f * per:(f + 1) * per]), p_ref), f
        check_decoded(to_host(out[f]), yg, Gf, g, f)


def test_fields_past_4gib_offsets():
    """Maximum-size addressing: two fields of 17,825,798 tokens (bf16, 4.56 GB
    each, so row offsets inside a field pass 2^32 bytes and the second field
    starts past them; the last block row is partial).  Sampled segments at
    the start, across the 4 GiB point and at the end are checked bit-exactly
    against the oracle, codes and decoded rows."""
    import torch
    L, KV, B, H = 1, 2, 1, 1
    T = (1 << 24) + (1 << 20) + 6
    Tcap = T + 2
    R, g = 4, 16
    x = kv_gpu(77, L, KV, B, H, T, Tcap, 0.95, 4, bf16=True)
    G = gauges_for(78, L, KV, H, g)
    shape = cg.make_shape(L, KV, B, H, T, Tcap, D, cg.CG_DTYPE_BF16)
    codec = cg.make_codec(cg.CG_BACKEND_ZFP, R)
    per = Tcap * D * R // 8
    pay = empty_u8(2 * per)
    out = torch.zeros_like(x)
    gauge = cg.make_gauge(g, to_dev(G))
    cg.cg_encode(shape, x, gauge, codec, 0, T, pay)
    cg.cg_decode(shape, pay, None, gauge, codec, 0, T, out)
    torch.cuda.synchronize()
    r_end = (T - 70) // 4 * 4
    for f in range(2):
        Gf = gauge_of_field(G, f, KV, B, H)
        for r0, n in ((0, 64), ((1 << 24) - 32, 96), (r_end, T - r_end)):
            xs = to_host(x[f, r0:r0 + n])
            n4 = (n + 3) // 4 * 4
            p_ref, yg = zfp_oracle_decoded(xs, Gf, g, R, n, n4)
            base = f * per + (r0 // 4) * 32 * 2 * R
            assert np.array_equal(to_host(pay[base:base + n4 // 4 * 32 * 2 * R]), p_ref), (f, r0)
            check_decoded(to_host(out[f, r0:r0 + n]), yg, Gf, g, (f, r0))
        assert not torch.any(out[f, T:].view(torch.int16) != 0)
    del x, out, pay
    torch.cuda.empty_cache()


def test_27b_class_full_size_sampled_fields():
    """The 27B-class codec workload at full size: 46 layers x K/V x 16 KV heads
    x 65536 tokens, bf16, g = 16, 3 b/v (12.35 G values, 24.7 GB), in one
    encode and one decode launch.  Sampled fields (layers 0, 23, 45; K and V;
    heads 0 and 15) bit-exact against the oracle, plus the last field."""
    import torch
    L, KV, B, H, T = 46, 2, 1, 16, 65536
    R, g = 3, 16
    x = kv_gpu(5, L, KV, B, H, T, T, 0.95, 4, bf16=True)
    G = gauges_for(105, L, KV, H, g)
    shape = cg.make_shape(L, KV, B, H, T, T, D, cg.CG_DTYPE_BF16)
    codec = cg.make_codec(cg.CG_BACKEND_ZFP, R)
    nbytes = cg.cg_encoded_bytes(shape, codec)[0]
    assert nbytes == L * KV * H * T * D * R // 8
    pay = empty_u8(nbytes)
    out = torch.empty_like(x)
    gauge = cg.make_gauge(g, to_dev(G))
    cg.cg_encode(shape, x, gauge, codec, 0, T, pay)
    cg.cg_decode(shape, pay, None, gauge, codec, 0, T, out)
    torch.cuda.synchronize()
    per = T * D * R // 8
    fields = [(l * KV + s) * H + h for l in (0, 23, 45) for s in (0, 1) for h in (0, 15)]
    fields.append(n_fields(L, KV, B, H) - 1)
    for f in sorted(set(fields)):
        xf = to_host(x[f])
        Gf = gauge_of_field(G, f, KV, B, H)
        p_ref, yg = zfp_oracle_decoded(xf, Gf, g, R, T, T)
        assert np.array_equal(to_host(pay[f * per:(f + 1) * per]), p_ref), f
        check_decoded(to_host(out[f]), yg, Gf, g, f)


@pytest.mark.parametrize("R", [3, 4, 8])
def test_full_head_gauge_zfp_fp32_bit_exact(R):
    """Full-head gauge (g = 128) with fp32 storage: the gauge runs as fp32
    matrix-core fmaf chains over k = 0..127 (the reading order of every
    group size), so payload and decoded cache are bit-exact against the
    oracle end to end.  The fp64 gauge is the tolerance reference for the
    1e-5 fp32 bar on the gauge and the inverse gauge."""
    t = __import__("torch")
    # 22 tiles: several 4-tile workgroup chunks, a ragged chunk, an 8-row last tile
    L, KV, B, H, T = 1, 2, 1, 2, 64 * 21 + 8
    x = kv_cpu(400 + R, L, KV, B, H, T, T, 0.95, 4, bf16=False)
    G = gauges_for(410, L, KV, H, 128)
    pay, out = run_zfp(x, G, 128, R, L, KV, B, H, T, T, False)
    per = T * D * R // 8
    worst_f, worst_i = 0.0, 0.0
    for f in range(n_fields(L, KV, B, H)):
        Gf = gauge_of_field(G, f, KV, B, H)
        xg = oracle.gauge_forward(x[f], Gf, 128)
        p_ref = oracle.zfp_encode_field(xg, R)
        assert np.array_equal(pay[f * per:(f + 1) * per], p_ref), f"payload mismatch in field {f}"
        dec = oracle.zfp_decode_field(p_ref, T, D, R)
        y = oracle.gauge_inverse(dec, Gf, 128)
        assert np.array_equal(out[f].view(np.uint32), y.view(np.uint32)), f"decoded mismatch in field {f}"
        G64 = Gf.astype(np.float64)
        worst_f = max(worst_f, rel_err(xg, oracle.gauge_forward_f64(x[f], G64, 128)))
        worst_i = max(worst_i, rel_err(out[f], oracle.gauge_inverse_f64(dec, G64, 128)))
    print(f"fp32 full-head gauge rel err {worst_f:.3e}, inverse gauge rel err {worst_i:.3e}")
    assert worst_f <= 1e-5 and worst_i <= 1e-5


@pytest.mark.parametrize("R", [3, 4, 8])
def test_dense_gauge_zfp_bf16_staged(R):
    """Full-head gauge (g = 128) with bf16 storage: the bf16 matrix-core
    gauge (one pass against the bf16 part of G) is not an fmaf chain, so
    parity is staged.  (1) The gauge, through cg_gauge_apply (the routine the
    fused kernels run), against the fp64 oracle within the one-pass bound of
    gpu_util.check_dense_forward; (2) the codes bit-exact against the oracle's
    coder applied to those gauged values; (3) the decoded cache within the
    bf16 bar (1e-2) of the oracle's fp64 inverse gauge of the oracle's decode
    of the same codes."""
    t = __import__("torch")
    L, KV, B, H, T = 1, 2, 1, 2, 64 * 21 + 8
    x = kv_cpu(400 + R, L, KV, B, H, T, T, 0.95, 4, bf16=True)
    G = gauges_for(410, L, KV, H, 128)
    pay, out = run_zfp(x, G, 128, R, L, KV, B, H, T, T, True)
    F = n_fields(L, KV, B, H)
    shape_in = cg.make_shape(L, KV, B, H, T, T, D, cg.CG_DTYPE_BF16)
    gauge = cg.make_gauge(128, to_dev(np.ascontiguousarray(G)))
    xg_d = t.zeros((F, T, D), dtype=t.float32, device="cuda")
    cg.cg_gauge_apply(shape_in, to_dev(x), gauge, 0, xg_d)
    t.cuda.synchronize()
    xg = to_host(xg_d)
    per = T * D * R // 8
    dec = np.zeros((F, T, D), np.float32)
    worst_g, worst_o = 0.0, 0.0
    for f in range(F):
        Gf = gauge_of_field(G, f, KV, B, H).astype(np.float64)
        worst_g = max(worst_g, check_dense_forward(xg[f], oracle.to_f32(x[f]), Gf, f))
        p_ref = oracle.zfp_encode_field(xg[f], R)
        assert np.array_equal(pay[f * per:(f + 1) * per], p_ref), f"payload mismatch in field {f}"
        dec[f] = oracle.zfp_decode_field(p_ref, T, D, R)
        ref = oracle.gauge_inverse_f64(dec[f], Gf, 128)
        worst_o = max(worst_o, rel_err(oracle.to_f32(out[f]), ref))
    print(f"bf16 dense gauge rel err {worst_g:.3e}; decoded cache vs fp64 inverse {worst_o:.3e}")
    assert worst_o <= 1e-2
