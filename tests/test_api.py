"""CPU-side contract of libcodecgauge.so: it loads, exports every symbol the
header declares, validates arguments on the host before any device work,
counts bytes exactly, and builds gauges with its own fp64 matrix exponential
(checked against the oracle's).  No device work is started here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from fixed_rate_compression_amd import binding as cg
from fixed_rate_compression_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "codec_gauge.h")).read()
    return sorted(set(re.findall(r"^(?:int|const char \*)\s*(cg_\w+)\(", txt, re.M)))


def test_library_exports_every_declared_symbol():
    L = cg.lib()
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(cg.EXPORTED)


def test_encoded_bytes_exact():
    # Llama-3-8B-class cache at 3, 4, 6 b/v: payload = rate x values / 8
    shape = cg.make_shape(32, 2, 1, 8, 32768, 32768, 128, cg.CG_DTYPE_BF16)
    N = 32 * 2 * 8 * 32768 * 128
    for R in (2, 3, 4, 6, 8):
        p, m, h = cg.cg_encoded_bytes(shape, cg.make_codec(cg.CG_BACKEND_ZFP, R))
        assert p == N * R // 8 and m == 0 and h == 64 * 32 * 2
        assert abs(8.0 * p / N - R) == 0.0


def test_encoded_bytes_quantizers():
    # block-uniform 3-bit, 64-token blocks: 8 B of metadata per block
    shape3 = cg.make_shape(32, 2, 1, 8, 131072, 131072, 128, cg.CG_DTYPE_BF16)
    p, m, _ = cg.cg_encoded_bytes(shape3, cg.make_codec(cg.CG_BACKEND_BLOCK_UNIFORM, 3, 64))
    N3 = 512 * 131072 * 128
    assert p == N3 * 3 // 8 and m == 512 * (131072 // 64) * 8
    # KIVI 4-bit, group 32, 128-token tail in bf16
    p, m, _ = cg.cg_encoded_bytes(shape3, cg.make_codec(cg.CG_BACKEND_KIVI, 4, 32, 128))
    assert p == 512 * ((131072 - 128) * 128 * 4 // 8 + 128 * 128 * 2)
    assert m == 512 * ((131072 - 128) * 128 // 32) * 8


@pytest.mark.parametrize("bad,code", [
    (dict(head_dim=64), cg.CG_E_UNSUPPORTED),
    (dict(kv=3), cg.CG_E_SHAPE),
    (dict(tokens=10, token_capacity=8), cg.CG_E_SHAPE),
    (dict(dtype=7), cg.CG_E_INVAL),
])
def test_shape_validation(bad, code):
    args = dict(layers=1, kv=2, batch=1, heads=2, tokens=64, token_capacity=64, head_dim=128,
                dtype=cg.CG_DTYPE_BF16)
    args.update(bad)
    shape = cg.CgShape(**args)
    with pytest.raises(cg.CodecGaugeError) as e:
        cg.cg_encoded_bytes(shape, cg.make_codec(cg.CG_BACKEND_ZFP, 4))
    assert e.value.code == code


def test_codec_and_row_validation_before_launch():
    shape = cg.make_shape(1, 2, 1, 2, 64, 64, 128, cg.CG_DTYPE_BF16)
    dummy = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    L = cg.lib()

    def enc(codec, t0, nt, gauge=cg.make_gauge(0), cap=1 << 30):
        return L.cg_encode(ctypes.byref(shape), dummy, ctypes.byref(gauge), ctypes.byref(codec),
                           t0, nt, dummy, cap, None, 0, None)

    assert enc(cg.make_codec(cg.CG_BACKEND_ZFP, 5), 0, 64) == cg.CG_E_UNSUPPORTED
    assert enc(cg.make_codec(cg.CG_BACKEND_ZFP, 4), 2, 60) == cg.CG_E_SHAPE
    assert enc(cg.make_codec(cg.CG_BACKEND_ZFP, 4), 0, 68) == cg.CG_E_SHAPE
    assert enc(cg.make_codec(cg.CG_BACKEND_ZFP, 4), 0, 64, cap=100) == cg.CG_E_SIZE
    assert enc(cg.make_codec(cg.CG_BACKEND_ZFP, 4), 0, 64, gauge=cg.make_gauge(12, np.zeros(1, np.float32))) == cg.CG_E_SHAPE
    assert enc(cg.make_codec(cg.CG_BACKEND_ZFP, 4), 0, 64, gauge=cg.CgGauge(16, None)) == cg.CG_E_INVAL
    # groups that divide head_dim but are not built are refused before any launch
    Gz = np.zeros(1, np.float32)
    assert enc(cg.make_codec(cg.CG_BACKEND_ZFP, 4), 0, 64, gauge=cg.make_gauge(4, Gz)) == cg.CG_E_UNSUPPORTED
    assert enc(cg.make_codec(cg.CG_BACKEND_ZFP, 4), 0, 64, gauge=cg.make_gauge(64, Gz)) == cg.CG_E_UNSUPPORTED
    assert enc(cg.make_codec(cg.CG_BACKEND_NONE, 4), 0, 64, gauge=cg.make_gauge(128, Gz)) == cg.CG_E_UNSUPPORTED
    assert "not built" in cg.cg_last_error()
    assert enc(cg.make_codec(9, 4), 0, 64) == cg.CG_E_INVAL
    assert "backend" in cg.cg_last_error()
    # zero rows is a no-op that launches nothing
    assert enc(cg.make_codec(cg.CG_BACKEND_ZFP, 4), 0, 0) == cg.CG_OK


def test_zfp_partial_block_row_only_at_the_end():
    # a zfp row range may end off a block-row boundary only at the field's
    # last valid token (the partial last block row is padded)
    shape = cg.make_shape(1, 2, 1, 2, 62, 64, 128, cg.CG_DTYPE_BF16)
    dummy = ctypes.c_void_p(16)
    L = cg.lib()
    codec = cg.make_codec(cg.CG_BACKEND_ZFP, 4)

    def enc(t0, nt):
        return L.cg_encode(ctypes.byref(shape), dummy, ctypes.byref(cg.make_gauge(0)),
                           ctypes.byref(codec), t0, nt, dummy, 1 << 30, None, 0, None)

    assert enc(0, 61) == cg.CG_E_SHAPE
    assert enc(0, 30) == cg.CG_E_SHAPE
    assert enc(2, 60) == cg.CG_E_SHAPE
    assert enc(0, 63) == cg.CG_E_SHAPE      # past the valid tokens


def test_gauge_from_skew_matches_oracle():
    for g in (2, 16, 32, 128):
        A = synth.gauge_params(g, 3, g)
        G = cg.cg_gauge_from_skew(A)
        ref = oracle.gauge_from_skew(A)
        assert np.max(np.abs(G.astype(np.float64) - ref)) <= 2.0 ** -24 * 2
        Gd = G.astype(np.float64)
        for b in range(3):
            assert np.max(np.abs(Gd[b].T @ Gd[b] - np.eye(g))) < g * 2.0 ** -23


def test_gauge_from_skew_closed_form_g2_large_angle():
    A = np.array([[[0.0, 3.0], [0.0, 0.0]]])
    G = cg.cg_gauge_from_skew(A)[0]
    a = 3.0
    ref = np.array([[np.cos(a), np.sin(a)], [-np.sin(a), np.cos(a)]])
    assert np.max(np.abs(G - ref)) < 1e-7


def test_header_layout():
    shape = cg.make_shape(2, 2, 1, 8, 100, 128, 128, cg.CG_DTYPE_BF16)
    h = cg.cg_write_header(shape, cg.make_codec(cg.CG_BACKEND_ZFP, 4), 1, 0)
    assert len(h) == 64 and h[:4] == b"CGKV"
    vals = np.frombuffer(h[4:48], np.int32)
    assert list(vals) == [1, 1, 4, 0, 0, 1, 1, 0, 1, 8, 128]
    assert list(np.frombuffer(h[48:64], np.int64)) == [100, 128]


def test_decode_gauged_and_gauge_heads_validation():
    dummy = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    L = cg.lib()
    codec = cg.make_codec(cg.CG_BACKEND_ZFP, 4)
    G = np.zeros(1, np.float32)

    def dec(shape, keep):
        return L.cg_decode_gauged(ctypes.byref(shape), dummy, 1 << 30, None, 0,
                                  ctypes.byref(cg.make_gauge(16, G)), ctypes.byref(codec), 0, 64,
                                  keep, dummy, None)

    s2 = cg.make_shape(1, 2, 1, 2, 64, 64, 128, cg.CG_DTYPE_BF16)
    s1 = cg.make_shape(1, 1, 1, 2, 64, 64, 128, cg.CG_DTYPE_BF16)
    assert dec(s2, 4) == cg.CG_E_INVAL and "keep" in cg.cg_last_error()
    assert dec(s2, -1) == cg.CG_E_INVAL
    assert dec(s1, cg.CG_KEEP_VALUES) == cg.CG_E_INVAL

    def heads(layer, kind, q_heads, rows, dtype=cg.CG_DTYPE_F32, x=16, y=1 << 40, g=16):
        return L.cg_gauge_heads(ctypes.byref(s2), ctypes.byref(cg.make_gauge(g, G)), layer, kind,
                                q_heads, rows, dtype, ctypes.c_void_p(x), ctypes.c_void_p(y), None)

    assert heads(1, 0, 8, 4) == cg.CG_E_SHAPE         # layer outside the cache
    assert heads(0, 2, 8, 4) == cg.CG_E_SHAPE         # kind outside the cache
    assert heads(0, 0, 3, 4) == cg.CG_E_SHAPE         # q_heads not a multiple of heads
    assert heads(0, 0, 8, -1) == cg.CG_E_SHAPE
    assert heads(0, 0, 8, 4, dtype=7) == cg.CG_E_INVAL
    assert heads(0, 0, 8, 4, x=4096, y=4096 + 1024) == cg.CG_E_INVAL   # overlapping x and y
    assert "overlap" in cg.cg_last_error()
    assert heads(0, 0, 8, 4, g=64) == cg.CG_E_UNSUPPORTED
    assert heads(0, 0, 8, 0) == cg.CG_OK               # no rows: nothing launched


def test_misaligned_device_pointers_are_refused():
    shape = cg.make_shape(1, 2, 1, 2, 64, 64, 128, cg.CG_DTYPE_BF16)
    L = cg.lib()
    codec = cg.make_codec(cg.CG_BACKEND_ZFP, 4)
    ok, odd = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 8)

    def enc(kv, pay):
        return L.cg_encode(ctypes.byref(shape), kv, ctypes.byref(cg.make_gauge(0)), ctypes.byref(codec),
                           0, 64, pay, 1 << 30, None, 0, None)

    def dec(pay, out):
        return L.cg_decode(ctypes.byref(shape), pay, 1 << 30, None, 0, ctypes.byref(cg.make_gauge(0)),
                           ctypes.byref(codec), 0, 64, out, None)

    assert enc(odd, ok) == cg.CG_E_INVAL and "aligned" in cg.cg_last_error()
    assert enc(ok, odd) == cg.CG_E_INVAL
    assert dec(odd, ok) == cg.CG_E_INVAL
    assert dec(ok, odd) == cg.CG_E_INVAL
    G = np.zeros(64, np.float32)
    bad_gauge = cg.CgGauge(16, ctypes.c_void_p(G.ctypes.data + 2))
    assert L.cg_encode(ctypes.byref(shape), ok, ctypes.byref(bad_gauge), ctypes.byref(codec), 0, 64,
                       ok, 1 << 30, None, 0, None) == cg.CG_E_INVAL
    # the consumer-side gauge needs element alignment only
    assert L.cg_gauge_heads(ctypes.byref(shape), ctypes.byref(cg.make_gauge(0)), 0, 0, 2, 1,
                            cg.CG_DTYPE_F32, ctypes.c_void_p(4098), ctypes.c_void_p(1 << 40),
                            None) == cg.CG_E_INVAL


def test_noalloc_decode_error_refuses_more_partials_than_its_scratch():
    """The allocation-free cg_decode_error_noalloc checks, on the host and
    before any device call, that the call's error partials fit the library's
    built-in scratch (2^20 fields of 64 tokens need 24 MiB > 16 MiB)."""
    shape = cg.make_shape(1024, 2, 1, 512, 64, 64, 128, cg.CG_DTYPE_BF16)
    codec = cg.make_codec(cg.CG_BACKEND_ZFP, 4)
    gauge = cg.make_gauge(0)
    need = cg.cg_decode_error_workspace_bytes(shape, gauge, codec, 0, 64)
    assert need > cg.CG_NOALLOC_SCRATCH_BYTES
    fake = 1 << 20   # never dereferenced: the size check comes first
    rc = cg.lib().cg_decode_error_noalloc(ctypes.byref(shape), fake, 1 << 40, None, 0,
                                          ctypes.byref(gauge), ctypes.byref(codec), 0, 64, fake,
                                          fake, fake, None)
    assert rc == cg.CG_E_SIZE
    assert "scratch" in cg.lib().cg_last_error().decode()
