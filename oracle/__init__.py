"""Codec-Gauge CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct CPU implementations of every step of the
Codec-Gauge KV-cache round trip ("Codec-Gauge: Learning Compression-Friendly
Gauges for Transformer KV Caches", arXiv 2607.20538, and its Chinese
translation).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library in ``fixed_rate_compression_amd`` and never imports
it.

Parts:
  * ``oracle_codec.c`` (loaded here through ctypes): fp32 gauge application,
    the zfp-style fixed-rate block coder, block-uniform and KIVI-style
    quantizers, bf16 conversion.
  * ``linalg.py``: fp64 matrix exponential and its Frechet derivative.
  * ``spectral.py``: fp64 token-channel DCT statistics and their gradient.

Every function here is pinned by the ``-m "not gpu"`` tests (closed forms,
library routines that are independent of this code, brute force,
invariants); none is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .linalg import expm, expm_frechet, gauge_from_skew  # noqa: F401
from .spectral import dct_matrix, radius_matrix, dct_stats_field  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_codec.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile oracle_codec.c with gcc (contraction off) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        sig = {
            "oracle_gauge_forward": [I64, I, I, P, P, P],
            "oracle_gauge_inverse": [I64, I, I, P, P, P],
            "oracle_zfp_encode_field": [I64, I64, I, I, P, P],
            "oracle_zfp_decode_field": [I64, I64, I, I, P, P],
            "oracle_zfp_encode_block": [P, I, P],
            "oracle_zfp_decode_block": [P, I, P],
            "oracle_bu_encode_field": [I64, I64, I, I, I, P, P, P],
            "oracle_bu_decode_field": [I64, I64, I, I, I, P, P, P],
            "oracle_kivi_encode_field": [I64, I, I, I, I, P, P, P],
            "oracle_kivi_decode_field": [I64, I, I, I, I, P, P, P],
            "oracle_unpack_codes": [I64, I, P, P],
            "oracle_bf16_to_f32_array": [I64, P, P],
            "oracle_f32_to_bf16_array": [I64, P, P],
            "oracle_sequency_order": [P],
            "oracle_fwd_lift4": [P],
            "oracle_inv_lift4": [P],
        }
        for name, args in {"oracle_zfp_block_words": [P, P, P],
                           "oracle_zfp_decode_block_words": [P, I, P, P]}.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# --------------------------------------------------------------------------
# storage format
# --------------------------------------------------------------------------

def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32, exact."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_bf16_to_f32_array(h.size, _p(h), _p(out))
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even."""
    x = _f32(x)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_bf16_array(x.size, _p(x), _p(out))
    return out


def to_f32(field: np.ndarray) -> np.ndarray:
    """Storage field (fp32, or bf16 held as uint16) -> fp32."""
    if field.dtype == np.uint16:
        return bf16_to_f32(field)
    return _f32(field)


def from_f32(x: np.ndarray, storage_dtype) -> np.ndarray:
    if np.dtype(storage_dtype) == np.uint16:
        return f32_to_bf16(x)
    return _f32(x)


# --------------------------------------------------------------------------
# gauge (arXiv page, gauge parameterization: X' = G X per group; inverse G^T)
# --------------------------------------------------------------------------

def gauge_forward(x: np.ndarray, G: np.ndarray | None, g: int) -> np.ndarray:
    """x [T, d] fp32, G [d/g, g, g] fp32; fmaf chain k = 0..g-1 from +0."""
    x = _f32(x)
    T, d = x.shape
    y = np.empty_like(x)
    if g == 0:
        y[...] = x
        return y
    Gc = _f32(G)
    assert Gc.shape == (d // g, g, g)
    lib().oracle_gauge_forward(T, d, g, _p(Gc), _p(x), _p(y))
    return y


def gauge_inverse(y: np.ndarray, G: np.ndarray | None, g: int) -> np.ndarray:
    """G^T per group; fmaf chain i = 0..g-1 from +0."""
    y = _f32(y)
    T, d = y.shape
    x = np.empty_like(y)
    if g == 0:
        x[...] = y
        return x
    Gc = _f32(G)
    assert Gc.shape == (d // g, g, g)
    lib().oracle_gauge_inverse(T, d, g, _p(Gc), _p(y), _p(x))
    return x


def gauge_forward_f64(x: np.ndarray, G: np.ndarray, g: int) -> np.ndarray:
    """Exact-as-possible fp64 reference of the gauge (tolerance reference)."""
    x = np.asarray(x, np.float64)
    if g == 0:
        return x.copy()
    T, d = x.shape
    xr = x.reshape(T, d // g, g)
    return np.einsum("rik,trk->tri", np.asarray(G, np.float64), xr).reshape(T, d)


def gauge_inverse_f64(y: np.ndarray, G: np.ndarray, g: int) -> np.ndarray:
    y = np.asarray(y, np.float64)
    if g == 0:
        return y.copy()
    T, d = y.shape
    yr = y.reshape(T, d // g, g)
    return np.einsum("rik,tri->trk", np.asarray(G, np.float64), yr).reshape(T, d)


def gauge_heads(x: np.ndarray, G_lk: np.ndarray | None, g: int, q_heads: int) -> np.ndarray:
    """Consumer side of recovery folded into the downstream projection
    ("Codec-Gauge", arXiv HTML, gauge-parameterization paragraph): with the
    cache kept gauged, q . (G^T k') = (G q) . k' and W_o G^T has rows G w.
    x [rows, q_heads*d] fp32 -> the forward gauge (fmaf chain, as
    gauge_forward) on every head segment, query head h taking the gauges
    G_lk[h // (q_heads // H)] of its KV head; G_lk [H, d/g, g, g]."""
    x = _f32(x)
    rows, width = x.shape
    d = width // q_heads
    y = np.empty_like(x)
    if g == 0:
        y[...] = x
        return y
    H = G_lk.shape[0]
    ratio = q_heads // H
    assert q_heads % H == 0 and width == q_heads * d
    for h in range(q_heads):
        seg = slice(h * d, (h + 1) * d)
        y[:, seg] = gauge_forward(np.ascontiguousarray(x[:, seg]), G_lk[h // ratio], g)
    return y


# --------------------------------------------------------------------------
# zfp-style fixed-rate coder
# --------------------------------------------------------------------------

def sequency_order() -> np.ndarray:
    out = np.zeros(16, np.int32)
    lib().oracle_sequency_order(_p(out))
    return out


def fwd_lift4(v) -> np.ndarray:
    a = np.ascontiguousarray(v, dtype=np.int32).copy()
    lib().oracle_fwd_lift4(_p(a))
    return a


def inv_lift4(v) -> np.ndarray:
    a = np.ascontiguousarray(v, dtype=np.int32).copy()
    lib().oracle_inv_lift4(_p(a))
    return a


def zfp_encode_block(v, R: int) -> np.ndarray:
    """16 fp32 values (v[4*j+i], j token, i channel) -> 2R bytes."""
    v = _f32(v).reshape(16)
    out = np.zeros(2 * R, np.uint8)
    lib().oracle_zfp_encode_block(_p(v), R, _p(out))
    return out


def zfp_decode_block(b, R: int) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    assert b.size >= 2 * R
    v = np.zeros(16, np.float32)
    lib().oracle_zfp_decode_block(_p(b), R, _p(v))
    return v


def zfp_block_words(v):
    """Steps 1-5 of one block: (nonzero, emax, negabinary words u[16] in
    total-sequency order)."""
    v = _f32(v).reshape(16)
    u = np.zeros(16, np.uint32)
    e = np.zeros(1, np.int32)
    nz = lib().oracle_zfp_block_words(_p(v), _p(u), _p(e))
    return bool(nz), int(e[0]), u


def zfp_decode_block_words(b, R: int):
    """Plane decoding of one block: (nonzero, emax, u[16])."""
    b = np.ascontiguousarray(b, dtype=np.uint8)
    assert b.size >= 2 * R
    u = np.zeros(16, np.uint32)
    e = np.zeros(1, np.int32)
    nz = lib().oracle_zfp_decode_block_words(_p(b), R, _p(u), _p(e))
    return bool(nz), int(e[0]), u


def zfp_field_bytes(T: int, d: int, R: int) -> int:
    return T * d * R // 8


def zfp_pad_rows(x: np.ndarray, end: int) -> np.ndarray:
    """Rows [0, end) of x with a partial last 4-row block row completed by
    repeating row end-1 (the reading used for fields whose token count is
    not a multiple of 4; the page does not say how partial blocks are
    filled)."""
    e4 = (end + 3) // 4 * 4
    xp = np.zeros((e4, x.shape[1]), np.float32)
    xp[:end] = x[:end]
    xp[end:e4] = x[end - 1]
    return xp


def zfp_encode_field(x: np.ndarray, R: int, t0: int = 0, nt: int | None = None,
                     out: np.ndarray | None = None, T_payload: int | None = None) -> np.ndarray:
    """x [T, d] fp32 (already gauged) -> payload bytes [T_payload*d*R/8]
    (T_payload: the field's row capacity, a multiple of 4; default T).
    Rows [t0, t0+nt) are encoded; t0 is a multiple of 4, and when t0+nt is
    not, the last block row is padded (zfp_pad_rows)."""
    x = _f32(x)
    T, d = x.shape
    if nt is None:
        nt = T - t0
    Tp = T if T_payload is None else T_payload
    assert Tp % 4 == 0 and d % 4 == 0 and t0 % 4 == 0
    if (t0 + nt) % 4:
        x = zfp_pad_rows(x, t0 + nt)
        nt = x.shape[0] - t0
    assert x.shape[0] % 4 == 0 and t0 + nt <= Tp
    if out is None:
        out = np.zeros(zfp_field_bytes(Tp, d, R), np.uint8)
    lib().oracle_zfp_encode_field(t0, nt, d, R, _p(x), _p(out))
    return out


def zfp_decode_field(payload: np.ndarray, T: int, d: int, R: int, t0: int = 0,
                     nt: int | None = None) -> np.ndarray:
    """payload of a field of T rows (T a multiple of 4) -> [T, d] with rows
    [t0, t0+nt) decoded (whole block rows are decoded; rows past t0+nt of a
    partial last block row are left zero)."""
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    if nt is None:
        nt = T - t0
    assert T % 4 == 0 and t0 % 4 == 0
    n4 = (nt + 3) // 4 * 4
    x = np.zeros((T, d), np.float32)
    lib().oracle_zfp_decode_field(t0, n4, d, R, _p(payload), _p(x))
    x[t0 + nt:t0 + n4] = 0.0
    return x


# --------------------------------------------------------------------------
# block-uniform and KIVI-style quantizers
# --------------------------------------------------------------------------

def bu_encode_field(x: np.ndarray, Bt: int, bits: int):
    x = _f32(x)
    T, d = x.shape
    assert T % Bt == 0
    nb = T // Bt
    payload = np.zeros(T * d * bits // 8, np.uint8)
    meta = np.zeros((nb, 2), np.float32)
    lib().oracle_bu_encode_field(0, T, d, Bt, bits, _p(x), _p(payload), _p(meta))
    return payload, meta


def bu_decode_field(payload, meta, T: int, d: int, Bt: int, bits: int) -> np.ndarray:
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    meta = _f32(meta)
    x = np.zeros((T, d), np.float32)
    lib().oracle_bu_decode_field(0, T, d, Bt, bits, _p(payload), _p(meta), _p(x))
    return x


def kivi_encode_field(x: np.ndarray, kind: int, group: int, bits: int, residual: int):
    """kind 0 = keys (per-channel ranges over `group` tokens), 1 = values
    (per-token ranges over `group` channels).  Returns (payload, meta, tail)
    where tail = the last `residual` gauged rows in fp32 (the caller stores
    them in the storage format)."""
    x = _f32(x)
    T, d = x.shape
    Tq = T - residual
    assert Tq >= 0 and Tq % group == 0 and d % group == 0
    payload = np.zeros(Tq * d * bits // 8, np.uint8)
    nmeta = (Tq // group) * d if kind == 0 else Tq * (d // group)
    meta = np.zeros((nmeta, 2), np.float32)
    lib().oracle_kivi_encode_field(Tq, d, kind, group, bits, _p(x), _p(payload), _p(meta))
    return payload, meta, x[Tq:].copy()


def kivi_decode_field(payload, meta, tail, T: int, d: int, kind: int, group: int,
                      bits: int, residual: int) -> np.ndarray:
    Tq = T - residual
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    meta = _f32(meta)
    x = np.zeros((T, d), np.float32)
    lib().oracle_kivi_decode_field(Tq, d, kind, group, bits, _p(payload), _p(meta), _p(x))
    x[Tq:] = tail
    return x


def unpack_codes(payload: np.ndarray, n: int, bits: int) -> np.ndarray:
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    out = np.zeros(n, np.uint32)
    lib().oracle_unpack_codes(n, bits, _p(payload), _p(out))
    return out


# --------------------------------------------------------------------------
# composed per-field round trips (gauge -> backend -> decode -> inverse)
# --------------------------------------------------------------------------

def zfp_roundtrip_field(field: np.ndarray, G, g: int, R: int):
    """Storage field [T, d] (fp32, or bf16 as uint16) -> (payload, recon in
    the storage format, gauged fp32 field, decoded gauged fp32 field)."""
    x = to_f32(field)
    xg = gauge_forward(x, G, g)
    payload = zfp_encode_field(xg, R)
    yg = zfp_decode_field(payload, x.shape[0], x.shape[1], R)
    y = gauge_inverse(yg, G, g)
    return payload, from_f32(y, field.dtype), xg, yg
