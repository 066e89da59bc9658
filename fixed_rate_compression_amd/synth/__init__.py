"""Seeded synthetic KV inputs (shared by the HIP path's tests/bench and the
oracle's tests).  Holds none of the method's arithmetic: only the value
model that stands in for real KV caches, which are not available here.

Value model (per field = one (layer, K/V, sequence, head) slab [T][d]):
  * channel scales sigma_c = exp(z_c), z_c ~ N(0, 1) (lognormal(0, 1));
  * `outliers` channels, chosen by a seeded permutation, scaled by 20;
  * AR(1) along tokens: y_0 = e_0, y_t = rho*y_{t-1} + sqrt(1-rho^2)*e_t,
    e_t ~ N(0, 1) independently per channel; x[t, c] = sigma_c * y[t, c];
  * generated in fp32 and rounded to bf16 (round-to-nearest-even) when the
    storage format is bf16.
Gauge parameters: A entries iid N(0, 0.1^2) (one g x g matrix per layer,
K/V, head and group).

Two generators implement the same model: `kv_field_cpu` (numpy, for CPU-side
tests and golden fixtures) and `generate_gpu` (a Philox4x32-10 + Box-Muller
HIP kernel in libcgsynth.so, for multi-GB inputs).  They draw different
random numbers; GPU-generated inputs reach the oracle as copies, so nothing
requires the two to agree.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SYNTH_SRC = os.path.join(_HERE, "synth.hip")
_SYNTH_LIB = os.path.join(_HERE, "libcgsynth.so")


def channel_scales(seed: int, field: int, d: int, outliers: int) -> np.ndarray:
    """sigma[d] (fp32) of one field."""
    rng = np.random.default_rng([int(seed), int(field), 7])
    sig = np.exp(rng.standard_normal(d))
    idx = rng.permutation(d)[:outliers]
    sig[idx] *= 20.0
    return sig.astype(np.float32)


def channel_scales_many(seed: int, fields, d: int, outliers: int) -> np.ndarray:
    return np.stack([channel_scales(seed, f, d, outliers) for f in fields])


def kv_field_cpu(seed: int, field: int, T: int, d: int, rho: float, outliers: int,
                 bf16: bool = False, scale_field: int | None = None) -> np.ndarray:
    """One field [T, d]: fp32, or bf16 bit patterns (uint16) if bf16."""
    from scipy.signal import lfilter

    sig = channel_scales(seed, field if scale_field is None else scale_field, d, outliers)
    rng = np.random.default_rng([int(seed), int(field), 11])
    e = rng.standard_normal((T, d))
    c = np.sqrt(1.0 - rho * rho)
    e[0] /= c                      # stationary start: y_0 = e_0
    y = lfilter([c], [1.0, -rho], e, axis=0)
    x = (y * sig[None, :].astype(np.float64)).astype(np.float32)
    if bf16:
        return f32_to_bf16_bits(x)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit patterns (input preparation)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    keep = u >> 16
    rest = u & 0xFFFF
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & 1) == 1))
    return (keep + up).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def gauge_params(seed: int, n: int, g: int) -> np.ndarray:
    """A [n, g, g] fp64, entries N(0, 0.1^2)."""
    rng = np.random.default_rng([int(seed), 101])
    return 0.1 * rng.standard_normal((n, g, g))


# --------------------------------------------------------------------------
# GPU generator (libcgsynth.so)
# --------------------------------------------------------------------------

def build(force: bool = True) -> str:
    if force or not os.path.exists(_SYNTH_LIB):
        tmp = _SYNTH_LIB + ".tmp"
        subprocess.check_call([
            "hipcc", "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-o", tmp, _SYNTH_SRC])
        os.replace(tmp, _SYNTH_LIB)
    return _SYNTH_LIB


_slib = None


def _synth_lib():
    global _slib
    if _slib is None:
        import torch  # noqa: F401  (bind to torch's HIP runtime, see binding.lib)
        if not os.path.exists(_SYNTH_LIB):
            raise RuntimeError("libcgsynth.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_SYNTH_LIB)
        L.cgsynth_generate.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                       ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_void_p]
        L.cgsynth_generate.restype = ctypes.c_int
        _slib = L
    return _slib


def generate_gpu(out, T: int, rho: float, seed: int, field_ids, scales, stream=None) -> None:
    """Fill the torch CUDA tensor `out` [n_fields, Tcap, d] (fp32 or bf16)
    with the value model: rows [0, T) of field f use Philox key
    (seed, field_ids[f]) and channel scales scales[f]."""
    import torch

    n_fields, Tcap, d = out.shape
    assert 0 <= T <= Tcap
    ids = torch.as_tensor(np.asarray(field_ids, np.int64), device=out.device)
    sc = torch.as_tensor(np.asarray(scales, np.float32), device=out.device).contiguous()
    assert sc.shape == (n_fields, d)
    dt = {torch.float32: 0, torch.bfloat16: 1}[out.dtype]
    if stream is None:
        stream = torch.cuda.current_stream(out.device).cuda_stream
    rc = _synth_lib().cgsynth_generate(out.data_ptr(), n_fields, Tcap, T, d, float(rho),
                                       int(seed) & 0xFFFFFFFF, ids.data_ptr(), sc.data_ptr(),
                                       dt, ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"cgsynth_generate failed ({rc})")
