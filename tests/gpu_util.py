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


def zfp_oracle_field(field, Gf, g, R, T, Tcap):
    """Oracle payload bytes of one field [Tcap, D] (rows [0,T) encoded, the
    rest left zero) and its decoded rows in the storage format."""
    x = oracle.to_f32(field[:T])
    xg = oracle.gauge_forward(x, Gf, g)
    payload = np.zeros(Tcap * D * R // 8, np.uint8)
    oracle.zfp_encode_field(xg, R, t0=0, nt=T, out=payload, T_payload=Tcap)
    yg = oracle.zfp_decode_field(payload, Tcap, D, R, t0=0, nt=T)[:T]
    y = oracle.gauge_inverse(yg, Gf, g)
    return payload, oracle.from_f32(y, field.dtype)


def payload_bytes(shape, codec):
    p, m, _ = cg.cg_encoded_bytes(shape, codec)
    return p, m


def empty_u8(n):
    return torch().zeros(max(int(n), 1), dtype=torch().uint8, device="cuda")
