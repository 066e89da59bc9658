"""The HIP library's block codec (csrc/zfp_block.hpp), compiled for the host,
against the oracle: the exact source the kernels run, checked bit-for-bit on
the CPU (encode streams, decoded values, random/corrupt streams) before any
GPU run."""
import ctypes
import os

import numpy as np
import pytest

import oracle
from fixed_rate_compression_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tests", "hostcheck", "libzfphost.so")
RATES = (1, 2, 3, 4, 5, 6, 7, 8, 12, 16)


@pytest.fixture(scope="module")
def hc():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__._build_hostcheck()
    L = ctypes.CDLL(LIB)
    L.hc_encode_block.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.hc_encode_block_general.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.hc_decode_block.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.hc_decode_block_general.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.hc_decode_block_lifted.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.hc_lift_matrix.argtypes = [ctypes.c_void_p]
    L.hc_decode_blocks.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    L.hc_encode_blocks.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    return L


def enc(L, v, R, general=False):
    v = np.ascontiguousarray(v, np.float32)
    o = np.zeros(2 * R, np.uint8)
    fn = L.hc_encode_block_general if general else L.hc_encode_block
    assert fn(v.ctypes.data, R, o.ctypes.data) == 0
    return o


def dec(L, b, R, general=False):
    b = np.ascontiguousarray(b, np.uint8)
    o = np.zeros(16, np.float32)
    fn = L.hc_decode_block_general if general else L.hc_decode_block
    assert fn(b.ctypes.data, R, o.ctypes.data) == 0
    return o


@pytest.mark.parametrize("R", RATES)
def test_kv_blocks_bit_exact(hc, R):
    x = synth.kv_field_cpu(1, R, 128, 128, 0.95, 4)
    for t in range(0, 128, 4):
        for c in range(0, 128, 4):
            v = x[t:t + 4, c:c + 4].reshape(16)
            b = oracle.zfp_encode_block(v, R)
            assert np.array_equal(enc(hc, v, R), b)
            assert np.array_equal(enc(hc, v, R, general=True), b)
            ref = oracle.zfp_decode_block(b, R).view(np.uint32)
            assert np.array_equal(dec(hc, b, R).view(np.uint32), ref)
            assert np.array_equal(dec(hc, b, R, general=True).view(np.uint32), ref)


@pytest.mark.parametrize("R", RATES)
def test_wide_range_and_special_blocks(hc, R):
    rng = np.random.default_rng(R)
    blocks = [(rng.standard_normal(16) * np.exp(4 * rng.standard_normal(16))).astype(np.float32)
              for _ in range(600)]
    blocks += [np.zeros(16, np.float32), np.full(16, -0.0, np.float32), np.full(16, 1e-42, np.float32),
               np.full(16, 3.0e38, np.float32), np.eye(4, dtype=np.float32).reshape(16)]
    for v in blocks:
        b = oracle.zfp_encode_block(v, R)
        assert np.array_equal(enc(hc, v, R), b)
        assert np.array_equal(enc(hc, v, R, general=True), b)
        ref = oracle.zfp_decode_block(b, R).view(np.uint32)
        assert np.array_equal(dec(hc, b, R).view(np.uint32), ref)
        assert np.array_equal(dec(hc, b, R, general=True).view(np.uint32), ref)


@pytest.mark.parametrize("R", RATES)
def test_random_streams(hc, R):
    rng = np.random.default_rng(100 + R)
    for _ in range(1500):
        b = rng.integers(0, 256, 2 * R).astype(np.uint8)
        ref = oracle.zfp_decode_block(b, R).view(np.uint32)
        assert np.array_equal(dec(hc, b, R).view(np.uint32), ref)
        assert np.array_equal(dec(hc, b, R, general=True).view(np.uint32), ref)


def dec_lifted(L, b, R):
    b = np.ascontiguousarray(b, np.uint8)
    o = np.zeros(16, np.float32)
    applied = L.hc_decode_block_lifted(b.ctypes.data, R, o.ctypes.data)
    assert applied in (0, 1)
    return o if applied else None


@pytest.mark.parametrize("R", RATES)
def test_biased_random_fields(hc, R):
    """Whole random fields (4096 blocks each) decode like the oracle's field
    decoder: uniform bits, mostly-0 bits (long runs of failed tests, many
    planes) and mostly-1 bits (early caps at coefficient 15, all sixteen
    coefficients significant), with the kernels' reconstruction choice and
    with the 32-plane one forced."""
    rng = np.random.default_rng(700 + R)
    T = 512
    nb = T // 4 * 32
    for p_one in (0.5, 0.15, 0.85):
        raw = np.packbits(rng.random(8 * nb * 2 * R) < p_one, bitorder="little")
        ref = oracle.zfp_decode_field(raw, T, 128, R)
        for general in (0, 1):
            v = np.zeros(16 * nb, np.float32)
            assert hc.hc_decode_blocks(raw.ctypes.data, nb, R, general, v.ctypes.data) == 0
            got = v.reshape(T // 4, 32, 4, 4).transpose(0, 2, 1, 3).reshape(T, 128)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (R, p_one, general)


@pytest.mark.parametrize("R", RATES)
def test_mixed_value_fields_encode(hc, R):
    """Whole fields (4096 blocks each) encode like the oracle's field
    encoder, with the kernels' plane-word path and with the 16x16
    transposes forced: Gaussian values under lognormal channel scales with
    sparse zeros, subnormal rows and rows near the top of the fp32 range."""
    rng = np.random.default_rng(900 + R)
    T = 512
    x = rng.standard_normal((T, 128)) * np.exp(3 * rng.standard_normal(128))
    x[rng.random((T, 128)) < 0.1] = 0.0
    x[32:64] *= 1e-41
    x[96:128] = x[96:128] / np.max(np.abs(x[96:128])) * 3e38
    x = x.astype(np.float32)
    ref = oracle.zfp_encode_field(x, R)
    v = np.ascontiguousarray(x.reshape(T // 4, 4, 32, 4).transpose(0, 2, 1, 3))
    nb = T // 4 * 32
    for general in (0, 1):
        out = np.zeros(nb * 2 * R, np.uint8)
        assert hc.hc_encode_blocks(v.ctypes.data, nb, R, general, out.ctypes.data) == 0
        assert np.array_equal(out, ref), (R, general)


def test_lift_matrix_inverts_the_forward_transform(hc):
    """The integer matrix of the lifted reconstruction, divided by 16, is the
    inverse of the separable forward transform F (x) F with Lindstrom's
    F = 1/16 [[4,4,4,4],[5,1,-1,-5],[-4,4,4,-4],[-2,6,-6,2]] (zfp paper,
    decorrelating transform), columns in total-sequency order."""
    a = np.zeros(256, np.int32)
    hc.hc_lift_matrix(a.ctypes.data)
    a = a.reshape(16, 16).astype(np.float64)
    F = np.array([[4, 4, 4, 4], [5, 1, -1, -5], [-4, 4, 4, -4], [-2, 6, -6, 2]], np.float64) / 16
    seq = [0, 1, 4, 5, 2, 8, 6, 9, 3, 12, 10, 7, 13, 11, 14, 15]
    a_pos = np.zeros_like(a)
    a_pos[:, seq] = a
    Fi = np.linalg.inv(F)
    assert np.abs(a_pos / 16 - np.kron(Fi, Fi)).max() < 1e-12
    assert np.abs(a).max() <= 127


@pytest.mark.parametrize("R", RATES)
def test_lifted_reconstruction_bit_exact(hc, R):
    """Where the lifted (matrix-core) reconstruction applies, it gives the
    oracle's values bit for bit; on KV data at 2-8 bits/value it applies to
    almost every block."""
    x = synth.kv_field_cpu(1, R, 128, 128, 0.95, 4)
    applied = total = 0
    for t in range(0, 128, 4):
        for c in range(0, 128, 4):
            b = oracle.zfp_encode_block(x[t:t + 4, c:c + 4].reshape(16), R)
            got = dec_lifted(hc, b, R)
            total += 1
            if got is not None:
                applied += 1
                assert np.array_equal(got.view(np.uint32), oracle.zfp_decode_block(b, R).view(np.uint32))
    if 2 <= R <= 4:
        assert applied > 0.9 * total, (applied, total)
    rng = np.random.default_rng(300 + R)
    blocks = [(rng.standard_normal(16) * np.exp(4 * rng.standard_normal(16))).astype(np.float32)
              for _ in range(400)]
    blocks += [np.zeros(16, np.float32), np.full(16, 1e-42, np.float32), np.full(16, 3.0e38, np.float32),
               np.full(16, 1e-37, np.float32), np.eye(4, dtype=np.float32).reshape(16)]
    streams = [oracle.zfp_encode_block(v, R) for v in blocks]
    streams += [rng.integers(0, 256, 2 * R).astype(np.uint8) for _ in range(1500)]
    for b in streams:
        got = dec_lifted(hc, b, R)
        if got is not None:
            assert np.array_equal(got.view(np.uint32), oracle.zfp_decode_block(b, R).view(np.uint32))
