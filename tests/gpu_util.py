"""Helpers shared by the GPU parity tests: seeded inputs on the device, and the
oracle applied field by field to host copies of the same inputs."""
import numpy as np

import oracle
from fixed_rate_compression_amd import binding as cg
from fixed_rate_compression_amd import synth

D = 128


def torch():
    import torch as _t
    return _t


def n_fields(L, KV, B, H):
    return L * KV * B * H


def gauges_for(seed, L, KV, H, g):
    """G fp32 [L, KV, H, D/g, g, g] from A ~ N(0, 0.1^2), built by the
    oracle's fp64 exp and rounded to fp32 (an input shared by both sides)."""
    if g == 0:
        return None
    A = synth.gauge_params(seed, L * KV * H * (D // g), g)
    return oracle.gauge_from_skew(A).astype(np.float32).reshape(L, KV, H, D // g, g, g)


def kv_cpu(seed, L, KV, B, H, T, Tcap, rho, outliers, bf16):
    """[fields, Tcap, D] host array (fp32 or bf16 bits), rows >= T zero."""
    F = n_fields(L, KV, B, H)
    out = np.zeros((F, Tcap, D), np.uint16 if bf16 else np.float32)
    for f in range(F):
        out[f, :T] = synth.kv_field_cpu(seed, f, T, D, rho, outliers, bf16=bf16)
    return out


def kv_gpu(seed, L, KV, B, H, T, Tcap, rho, outliers, bf16):
    """Same value model generated on the device (Philox); returns a torch
    tensor [fields, Tcap, D] (bfloat16 or float32)."""
    t = torch()
    F = n_fields(L, KV, B, H)
    dt = t.bfloat16 if bf16 else t.float32
    x = t.zeros((F, Tcap, D), dtype=dt, device="cuda")
    scales = synth.channel_scales_many(seed, range(F), D, outliers)
    synth.generate_gpu(x, T, rho, seed, np.arange(F), scales)
    return x


def to_dev(a):
    t = torch()
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16).copy()).view(t.bfloat16).cuda()
    return t.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(x):
    """device tensor -> numpy (bf16 as uint16 bits)."""
    t = torch()
    c = x.detach().cpu().contiguous()
    if c.dtype == t.bfloat16:
        return c.view(t.int16).numpy().view(np.uint16)
    if c.dtype == t.uint8:
        return c.numpy()
    return c.numpy()


def gauge_of_field(G, f, KV, B, H):
    """G [L,KV,H,R,g,g] -> the [R,g,g] set of field f (fields are L,KV,B,H)."""
    if G is None:
        return None
    h = f % H
    ls = f // (B * H)
    l, s = divmod(ls, KV)
    return G[l, s, h]


def zfp_oracle_decoded(field, Gf, g, R, T, Tcap):
    """Oracle payload bytes of one field [Tcap, D] (rows [0,T) encoded, the
    rest left zero) and its decoded rows before the inverse gauge (fp32)."""
    x = oracle.to_f32(field[:T])
    xg = oracle.gauge_forward(x, Gf, g)
    payload = np.zeros(Tcap * D * R // 8, np.uint8)
    oracle.zfp_encode_field(xg, R, t0=0, nt=T, out=payload, T_payload=Tcap)
    yg = oracle.zfp_decode_field(payload, Tcap, D, R, t0=0, nt=T)[:T]
    return payload, yg


def zfp_oracle_field(field, Gf, g, R, T, Tcap):
    """Oracle payload bytes of one field and its decoded rows in the storage
    format."""
    payload, yg = zfp_oracle_decoded(field, Gf, g, R, T, Tcap)
    return payload, oracle.from_f32(oracle.gauge_inverse(yg, Gf, g), field.dtype)


def check_dense_forward(xg, x, Gf, where=None):
    """The full-head gauge of bf16 tiles (one pass of bf16 matrix-core products
    against the round-to-nearest bf16 part of the gauge: the tile values are
    bf16 already) against fp64: every element within 2^-8 sum_k |G_ck| |x_k|
    (the bf16 rounding of G contributes at most 2^-9 of it, the fp32 sums
    about 2^-17), and the 1e-2 bar of bf16 I/O as max|err| / max|ref|.
    Returns that relative error."""
    x64 = np.asarray(x, np.float64)
    G64 = np.asarray(Gf, np.float64)
    ref = oracle.gauge_forward_f64(x64, G64, 128)
    mag = oracle.gauge_forward_f64(np.abs(x64), np.abs(G64), 128)
    err = np.abs(np.asarray(xg, np.float64) - ref)
    assert np.all(err <= 2.0 ** -8 * mag), (where, float(np.max(err / np.maximum(mag, 1e-300))))
    rel = float(np.max(err) / max(np.max(np.abs(ref)), 1e-30))
    assert rel <= 1e-2, (where, rel)
    return rel


def check_dense_inverse(got, deq, Gf, where=None, row_min=None):
    """Decoded bf16 rows of the full-head decoders against the fp64 inverse
    gauge of the oracle's dequantized values `deq`.  The decoders form the
    product in fp16 with fp32 sums: KIVI-style rows scaled by a power of two
    into fp16's range (each value and each gauge entry within 2^-11 of
    itself), so the unrounded result is within 2^-10 sum_k |G_kc| |x_k|.
    Block-uniform rows (`row_min`: the minimum of each row's block) multiply
    the exact codes q = (x - min) / step and add min * colsum(G) after the
    product, so there the gauge rounding scales with sum |G| |x - min| and
    the fp32 sums with |min| sum |G|: the sums of the bound run over
    |x| + |x - min|.  The bf16 rounding adds at most 2^-8 of the value.
    Every element must satisfy |got - ref| <= 2^-8 |ref| + 2^-9 sum |G| m
    (m = |x|, or |x| + |x - min|), and the 1e-2 bar as max|err| / max|ref|.
    Returns that relative error."""
    x64 = np.asarray(deq, np.float64)
    G64 = np.asarray(Gf, np.float64)
    ref = oracle.gauge_inverse_f64(x64, G64, 128)
    m = np.abs(x64)
    if row_min is not None:
        m = m + np.abs(x64 - np.asarray(row_min, np.float64).reshape(-1, 1))
    mag = oracle.gauge_inverse_f64(m, np.abs(G64), 128)
    val = oracle.to_f32(got).astype(np.float64)
    err = np.abs(val - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -9 * mag
    assert np.all(err <= bound), (where, float(np.max(err / np.maximum(bound, 1e-300))))
    rel = float(np.max(err) / max(np.max(np.abs(ref)), 1e-30))
    assert rel <= 1e-2, (where, rel)
    return rel


def split_inverse(storage_dtype, g):
    """True where the library's decoders apply the inverse gauge as
    split-precision bf16 matrix-core products: bf16 storage with g = 16 or
    32 (elsewhere they evaluate the oracle's fmaf chains)."""
    return np.dtype(storage_dtype) == np.uint16 and g in (16, 32)


def check_decoded(got, yg, Gf, g, where=None):
    """Decoded rows `got` (storage format) against the oracle's decoded values
    yg (fp32, before the inverse gauge).

    fmaf-chain decoders: bit-exact.  Split-precision decoders (bf16 storage,
    g = 16 / 32; the pages' bar for bf16 I/O is 1e-2 relative): each product
    x G is formed from bf16 parts (x = x_hi + x_lo with |x - x_hi - x_lo| <=
    2^-16 |x|, G likewise within 2^-18 |G|, the dropped x_lo G_lo term
    <= 2^-16 |x G|) and summed in fp32, so the unrounded result is within
    2^-14.5 sum_k |G_kc| |x_k| of the exact one, and the bf16 rounding adds at
    most 2^-8 of the value.  Every element must satisfy
        |got - ref| <= 2^-8 |ref| + 2^-13 sum_k |G_kc| |x_k|
    (ref the fp64 inverse gauge of yg), the normwise relative error must be
    within the 1e-2 bar, and at least 90 % of the elements must equal the
    oracle's fmaf-chain result bit for bit (typically 97-99.9 %: a bf16
    rounding of the two results differs only near a rounding boundary)."""
    if not split_inverse(got.dtype, g):
        ref = oracle.from_f32(oracle.gauge_inverse(yg, Gf, g), got.dtype)
        assert np.array_equal(got.view(np.uint32 if got.dtype == np.float32 else np.uint16),
                              ref.view(np.uint32 if ref.dtype == np.float32 else np.uint16)), where
        return
    ref = oracle.gauge_inverse_f64(yg, Gf, g)
    mag = oracle.gauge_inverse_f64(np.abs(yg.astype(np.float64)), np.abs(np.asarray(Gf, np.float64)), g)
    val = oracle.bf16_to_f32(got).astype(np.float64)
    err = np.abs(val - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -13 * mag
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    assert np.all(err <= bound), (where, worst)
    rel = float(np.linalg.norm(val - ref) / max(np.linalg.norm(ref), 1e-300))
    assert rel <= 1e-2, (where, rel)
    chain = oracle.f32_to_bf16(oracle.gauge_inverse(yg, Gf, g))
    same = float(np.mean(got == chain)) if got.size else 1.0
    assert same >= 0.90, (where, same)


def payload_bytes(shape, codec):
    p, m, _ = cg.cg_encoded_bytes(shape, codec)
    return p, m


def empty_u8(n):
    return torch().zeros(max(int(n), 1), dtype=torch().uint8, device="cuda")
