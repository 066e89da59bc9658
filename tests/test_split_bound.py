"""The error bounds that the GPU tests apply to the decoders' reduced-precision
inverse gauges, checked on the CPU against models of that arithmetic:
- g = 16 / 32 with bf16 storage (gpu_util.check_decoded): decoded values
  split into a truncated bf16 part and the bf16-rounded remainder, gauge
  entries into two round-to-nearest bf16 parts, the products hi*hi + hi*lo +
  lo*hi (+ lo*lo at g = 16) summed (here exactly, in fp64) and rounded to
  fp32, then to bf16;
- the full-head gauge with bf16 storage (gpu_util.check_dense_inverse):
  rows scaled by a power of two into fp16, times the fp16 part of G
  (KIVI-style), or the exact codes times the fp16 part of G, then
  step * product + min * colsum(G) (block-uniform)."""
import numpy as np
import pytest

import oracle
from fixed_rate_compression_amd import synth


def bf16_rne(a):
    return oracle.bf16_to_f32(oracle.f32_to_bf16(a.astype(np.float32))).astype(np.float64)


def bf16_trunc(a):
    return (a.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


def split_inverse_model(y, G, g):
    yh = bf16_trunc(y)
    yl = bf16_rne(y.astype(np.float64) - yh)
    Gh = bf16_rne(G)
    Gl = bf16_rne(G.astype(np.float64) - Gh)
    acc = (oracle.gauge_inverse_f64(yh, Gh, g) + oracle.gauge_inverse_f64(yh, Gl, g)
           + oracle.gauge_inverse_f64(yl, Gh, g))
    if g == 16:
        acc += oracle.gauge_inverse_f64(yl, Gl, g)
    acc = acc.astype(np.float32)
    return acc.astype(np.float64), oracle.bf16_to_f32(oracle.f32_to_bf16(acc)).astype(np.float64)


@pytest.mark.parametrize("g", [16, 32])
def test_bound_holds_on_decoded_and_wide_values(g):
    G = oracle.gauge_from_skew(synth.gauge_params(7 + g, 128 // g, g)).astype(np.float32)
    x = synth.kv_field_cpu(3, g, 256, 128, 0.95, 4)
    y = oracle.zfp_decode_field(oracle.zfp_encode_field(oracle.gauge_forward(x, G, g), 4), 256, 128, 4)
    rng = np.random.default_rng(g)
    wide = (rng.standard_normal((256, 128)) * np.exp(3 * rng.standard_normal((256, 128)))).astype(np.float32)
    for v in (y, wide):
        acc, got = split_inverse_model(v, G, g)
        ref = oracle.gauge_inverse_f64(v, G, g)
        mag = oracle.gauge_inverse_f64(np.abs(v.astype(np.float64)), np.abs(G.astype(np.float64)), g)
        # the unrounded sum: within 2^-14.5 of sum |G||x| (split residuals and
        # the dropped lo*lo term), the margin the 2^-13 term leaves for fp32
        # accumulation order
        assert np.max(np.abs(acc - ref) / np.maximum(mag, 1e-300)) <= 2.0 ** -14.5
        bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -13 * mag
        assert np.all(np.abs(got - ref) <= bound)


def f16_scaled_inverse_model(x, G):
    """fp16 form of the full-head decoders: each row scaled by 2^k so that its
    largest magnitude lies in [2^13, 2^14), rounded to fp16, times the fp16
    part of G (sums exact here), scaled back."""
    x = np.asarray(x, np.float32)
    m = np.max(np.abs(x), axis=1, keepdims=True)
    e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
    k = np.where(m > 0, np.minimum(13 - e, 127), 0)
    xs = (x.astype(np.float64) * np.exp2(k)).astype(np.float16).astype(np.float64)
    G16 = np.asarray(G, np.float32).astype(np.float16).astype(np.float64)
    return oracle.gauge_inverse_f64(xs, G16, 128) * np.exp2(-k)


def test_fp16_dense_inverse_bound():
    """The unrounded fp16 product stays within 2^-10 sum |G||x| (the bound
    gpu_util.check_dense_inverse builds on), on dequantized-like rows and on
    rows of very different scales."""
    G = oracle.gauge_from_skew(synth.gauge_params(11, 1, 128)).astype(np.float32)
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((256, 128)).astype(np.float32)
    rows *= np.exp2(rng.integers(-40, 40, size=(256, 1))).astype(np.float32)
    rows[:8] = 0.0
    rows[8:16, :64] = 0.0
    for x in (rows, np.round(rows * 7) / 7):
        got = f16_scaled_inverse_model(x, G)
        ref = oracle.gauge_inverse_f64(x, G, 128)
        mag = oracle.gauge_inverse_f64(np.abs(x.astype(np.float64)), np.abs(G.astype(np.float64)), 128)
        assert np.all(np.abs(got - ref) <= 2.0 ** -10 * mag)


def test_fp16_block_uniform_inverse_bound():
    """Block-uniform form: codes q (exact in fp16) times the fp16 part of G,
    then step * (q G) + min * colsum(G).  Within 2^-10 sum |G| (|x| + |x - min|)
    of the fp64 inverse gauge of the fp32 dequantized values min + q step,
    also where a narrow range sits far from zero (the products of min and
    the column sums cancel)."""
    G = oracle.gauge_from_skew(synth.gauge_params(12, 1, 128)).astype(np.float32)
    G16 = G.astype(np.float16).astype(np.float64)
    cs = G.astype(np.float64).reshape(128, 128).sum(axis=0)
    rng = np.random.default_rng(6)
    for bits in (3, 6, 8):
        q = rng.integers(0, 1 << bits, size=(256, 128)).astype(np.float64)
        mn = (rng.standard_normal((256, 1)) * np.exp2(rng.integers(-20, 20, size=(256, 1)))).astype(np.float32)
        sc = (np.abs(rng.standard_normal((256, 1))) * np.exp2(rng.integers(-30, 10, size=(256, 1)))).astype(np.float32)
        mn[:16] = -100.0
        sc[:16] = 1e-3
        deq = (mn.astype(np.float64) + q * sc).astype(np.float32).astype(np.float64)
        got = sc.astype(np.float64) * oracle.gauge_inverse_f64(q, G16, 128) + mn.astype(np.float64) * cs
        ref = oracle.gauge_inverse_f64(deq, G.astype(np.float64), 128)
        m = np.abs(deq) + np.abs(deq - mn.astype(np.float64))
        mag = oracle.gauge_inverse_f64(m, np.abs(G.astype(np.float64)), 128)
        assert np.all(np.abs(got - ref) <= 2.0 ** -10 * mag), bits
