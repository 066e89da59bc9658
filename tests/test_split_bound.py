"""The error bound that the GPU tests apply to split-precision inverse gauges
(bf16 storage, g = 16 / 32; gpu_util.check_decoded), checked on the CPU
against a model of that arithmetic: decoded values split into a truncated
bf16 part and the bf16-rounded remainder, gauge entries into two
round-to-nearest bf16 parts, the products hi*hi + hi*lo + lo*hi (+ lo*lo at
g = 16) summed (here exactly, in fp64) and rounded to fp32, then to bf16."""
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
