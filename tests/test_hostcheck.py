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
    L.hc_decode_block.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return L


def enc(L, v, R):
    v = np.ascontiguousarray(v, np.float32)
    o = np.zeros(2 * R, np.uint8)
    assert L.hc_encode_block(v.ctypes.data, R, o.ctypes.data) == 0
    return o


def dec(L, b, R):
    b = np.ascontiguousarray(b, np.uint8)
    o = np.zeros(16, np.float32)
    assert L.hc_decode_block(b.ctypes.data, R, o.ctypes.data) == 0
    return o


@pytest.mark.parametrize("R", RATES)
def test_kv_blocks_bit_exact(hc, R):
    x = synth.kv_field_cpu(1, R, 128, 128, 0.95, 4)
    for t in range(0, 128, 4):
        for c in range(0, 128, 4):
            v = x[t:t + 4, c:c + 4].reshape(16)
            b = oracle.zfp_encode_block(v, R)
            assert np.array_equal(enc(hc, v, R), b)
            assert np.array_equal(dec(hc, b, R).view(np.uint32), oracle.zfp_decode_block(b, R).view(np.uint32))


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
        assert np.array_equal(dec(hc, b, R).view(np.uint32), oracle.zfp_decode_block(b, R).view(np.uint32))


@pytest.mark.parametrize("R", RATES)
def test_random_streams(hc, R):
    rng = np.random.default_rng(100 + R)
    for _ in range(1500):
        b = rng.integers(0, 256, 2 * R).astype(np.uint8)
        assert np.array_equal(dec(hc, b, R).view(np.uint32), oracle.zfp_decode_block(b, R).view(np.uint32))
