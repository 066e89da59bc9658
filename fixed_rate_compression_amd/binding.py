"""Thin ctypes binding of libcodecgauge.so (include/codec_gauge.h).

Argument marshalling only: the functions keep the C names, take torch CUDA
tensors (or numpy arrays for host arguments), pass raw pointers plus the
current HIP stream, and raise on a negative return code.  All computation
happens in the HIP library; if it is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libcodecgauge.so")

CG_OK = 0
CG_E_INVAL, CG_E_SHAPE, CG_E_UNSUPPORTED, CG_E_SIZE, CG_E_HIP, CG_E_INTERNAL = -1, -2, -3, -4, -5, -6
CG_DTYPE_F32, CG_DTYPE_BF16 = 0, 1
CG_BACKEND_NONE, CG_BACKEND_ZFP, CG_BACKEND_BLOCK_UNIFORM, CG_BACKEND_KIVI = 0, 1, 2, 3
CG_HEADER_BYTES = 64

EXPORTED = ["cg_encoded_bytes", "cg_encode", "cg_decode", "cg_decode_gauged", "cg_roundtrip",
            "cg_gauge_fit_stats", "cg_gauge_fit_grad", "cg_stats_workspace_bytes", "cg_gauge_from_skew",
            "cg_gauge_apply", "cg_write_header", "cg_decode_error_workspace_bytes",
            "cg_decode_error", "cg_decode_error_noalloc", "cg_cache_error_summary", "cg_adamw_update", "cg_gauge_control",
            "cg_second_moment_workspace_bytes", "cg_second_moment", "cg_gauge_grad", "cg_gauge_heads",
            "cg_last_error"]

CG_KEEP_KEYS, CG_KEEP_VALUES = 1, 2
CG_NOALLOC_SCRATCH_BYTES = 16 << 20
CG_CONTROL_IDENTITY, CG_CONTROL_HADAMARD, CG_CONTROL_DCT, CG_CONTROL_ORTHONORMALIZE, CG_CONTROL_KLT = range(5)


class CgShape(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("kv", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("tokens", ctypes.c_int64),
                ("token_capacity", ctypes.c_int64), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class CgGauge(ctypes.Structure):
    _fields_ = [("group", ctypes.c_int32), ("G", ctypes.c_void_p)]


class CgCodec(ctypes.Structure):
    _fields_ = [("backend", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("block_tokens", ctypes.c_int32), ("residual_tokens", ctypes.c_int32)]


class CgFieldError(ctypes.Structure):
    _fields_ = [("sse", ctypes.c_double), ("ref_ss", ctypes.c_double), ("max_abs", ctypes.c_double),
                ("values", ctypes.c_double)]


class CgCacheError(ctypes.Structure):
    _fields_ = [("mse", ctypes.c_double), ("nrmse", ctypes.c_double), ("key_nrmse", ctypes.c_double),
                ("value_nrmse", ctypes.c_double), ("max_abs", ctypes.c_double),
                ("values", ctypes.c_double)]


class CgStats(ctypes.Structure):
    _fields_ = [("L_freq", ctypes.c_double), ("L_rate", ctypes.c_double), ("L", ctypes.c_double),
                ("sum_E", ctypes.c_double)]


class CodecGaugeError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch loads its bundled HIP runtime under the name "libamdhip64.so";
        # importing it first lets this library's libamdhip64.so.7 dependency
        # resolve (by soname) to that same runtime instead of a second copy
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        SP, GP, CP = ctypes.POINTER(CgShape), ctypes.POINTER(CgGauge), ctypes.POINTER(CgCodec)
        U64P = ctypes.POINTER(ctypes.c_uint64)
        sig = {
            "cg_encoded_bytes": [SP, CP, U64P, U64P, U64P],
            "cg_encode": [SP, P, GP, CP, I64, I64, P, U64, P, U64, P],
            "cg_decode": [SP, P, U64, P, U64, GP, CP, I64, I64, P, P],
            "cg_decode_gauged": [SP, P, U64, P, U64, GP, CP, I64, I64, I32, P, P],
            "cg_gauge_heads": [SP, GP, I32, I32, I32, I64, I32, P, P, P],
            "cg_roundtrip": [SP, P, GP, CP, P, U64, P, U64, P, P],
            "cg_gauge_fit_stats": [SP, P, I32, P, I32, ctypes.c_float, ctypes.c_float,
                                   ctypes.c_float, P, ctypes.c_size_t, P, P, P],
            "cg_gauge_fit_grad": [SP, P, I32, P, I32, ctypes.c_float, ctypes.c_float,
                                   ctypes.c_float, P, ctypes.c_size_t, P, P, P],
            "cg_stats_workspace_bytes": [SP, I32, I32, ctypes.POINTER(ctypes.c_size_t)],
            "cg_gauge_from_skew": [I64, I32, P, P],
            "cg_gauge_apply": [SP, P, GP, I32, P, P],
            "cg_write_header": [SP, CP, I32, I32, P, U64],
            "cg_decode_error_workspace_bytes": [SP, GP, CP, I64, I64, ctypes.POINTER(ctypes.c_size_t)],
            "cg_decode_error": [SP, P, U64, P, U64, GP, CP, I64, I64, P, P, P, ctypes.c_size_t, P, P],
            "cg_decode_error_noalloc": [SP, P, U64, P, U64, GP, CP, I64, I64, P, P, P, P],
            "cg_cache_error_summary": [SP, P, ctypes.POINTER(CgCacheError)],
            "cg_adamw_update": [I64, P, P, P, P, I64, ctypes.c_double, ctypes.c_double,
                                ctypes.c_double, ctypes.c_double, ctypes.c_double],
            "cg_gauge_control": [I32, I64, I32, P, P],
            "cg_second_moment_workspace_bytes": [SP, I32, ctypes.POINTER(ctypes.c_size_t)],
            "cg_second_moment": [SP, P, I32, P, ctypes.c_size_t, P, P],
            "cg_gauge_grad": [I64, I32, P, P, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.cg_last_error.argtypes = []
        L.cg_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(fn, rc):
    if rc != CG_OK:
        raise CodecGaugeError(fn, rc, lib().cg_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):          # a raw device address (e.g. a window inside a tensor)
        return t
    if isinstance(t, np.ndarray):
        assert t.flags["C_CONTIGUOUS"]
        return t.ctypes.data
    assert t.is_contiguous(), "tensors must be contiguous"
    return t.data_ptr()


def _nbytes(t):
    if t is None:
        return 0
    if isinstance(t, np.ndarray):
        return t.nbytes
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_shape(layers, kv, batch, heads, tokens, token_capacity=None, head_dim=128,
               dtype=CG_DTYPE_BF16) -> CgShape:
    return CgShape(layers, kv, batch, heads, tokens,
                   tokens if token_capacity is None else token_capacity, head_dim, dtype)


def make_gauge(group: int, G=None) -> CgGauge:
    gg = CgGauge(group, _ptr(G) if G is not None else None)
    gg._keep = G      # the struct holds a raw pointer: keep the tensor alive with it
    return gg


def make_codec(backend, bits=4, block_tokens=0, residual_tokens=0) -> CgCodec:
    return CgCodec(backend, bits, block_tokens, residual_tokens)


def cg_encoded_bytes(shape: CgShape, codec: CgCodec):
    p, m, h = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    _check("cg_encoded_bytes", lib().cg_encoded_bytes(ctypes.byref(shape), ctypes.byref(codec),
                                                      ctypes.byref(p), ctypes.byref(m),
                                                      ctypes.byref(h)))
    return p.value, m.value, h.value


def cg_encode(shape, kv, gauge, codec, t0, nt, payload, meta=None, stream=None):
    _check("cg_encode", lib().cg_encode(ctypes.byref(shape), _ptr(kv), ctypes.byref(gauge),
                                        ctypes.byref(codec), t0, nt, _ptr(payload),
                                        _nbytes(payload), _ptr(meta), _nbytes(meta),
                                        _stream(stream)))


def cg_decode(shape, payload, meta, gauge, codec, t0, nt, kv_out, stream=None):
    _check("cg_decode", lib().cg_decode(ctypes.byref(shape), _ptr(payload), _nbytes(payload),
                                        _ptr(meta), _nbytes(meta), ctypes.byref(gauge),
                                        ctypes.byref(codec), t0, nt, _ptr(kv_out),
                                        _stream(stream)))


def cg_decode_gauged(shape, payload, meta, gauge, codec, t0, nt, keep, kv_out, stream=None):
    """cg_decode leaving the kinds in `keep` (CG_KEEP_KEYS | CG_KEEP_VALUES) gauged."""
    _check("cg_decode_gauged", lib().cg_decode_gauged(
        ctypes.byref(shape), _ptr(payload), _nbytes(payload), _ptr(meta), _nbytes(meta),
        ctypes.byref(gauge), ctypes.byref(codec), t0, nt, keep, _ptr(kv_out), _stream(stream)))


def cg_gauge_heads(shape, gauge, layer, kind, q_heads, rows, dtype, x, y, stream=None):
    """Forward gauge of (layer, kind) on the head segments of x [rows][q_heads*d] -> y."""
    _check("cg_gauge_heads", lib().cg_gauge_heads(
        ctypes.byref(shape), ctypes.byref(gauge), layer, kind, q_heads, rows, dtype, _ptr(x),
        _ptr(y), _stream(stream)))


def cg_decode_error_workspace_bytes(shape, gauge, codec, t0, nt):
    b = ctypes.c_size_t()
    _check("cg_decode_error_workspace_bytes", lib().cg_decode_error_workspace_bytes(
        ctypes.byref(shape), ctypes.byref(gauge), ctypes.byref(codec), t0, nt, ctypes.byref(b)))
    return b.value


def cg_decode_error(shape, payload, meta, gauge, codec, t0, nt, kv_out, kv_ref, workspace, err,
                    stream=None):
    """err: device float64 tensor [n_fields, 4] (sse, ref_ss, max_abs, values)."""
    _check("cg_decode_error", lib().cg_decode_error(
        ctypes.byref(shape), _ptr(payload), _nbytes(payload), _ptr(meta), _nbytes(meta),
        ctypes.byref(gauge), ctypes.byref(codec), t0, nt, _ptr(kv_out), _ptr(kv_ref),
        _ptr(workspace), _nbytes(workspace), _ptr(err), _stream(stream)))


def cg_decode_error_noalloc(shape, payload, meta, gauge, codec, t0, nt, kv_out, kv_ref, err,
                            stream=None):
    """cg_decode_error with the library's built-in device scratch (no workspace)."""
    _check("cg_decode_error_noalloc", lib().cg_decode_error_noalloc(
        ctypes.byref(shape), _ptr(payload), _nbytes(payload), _ptr(meta), _nbytes(meta),
        ctypes.byref(gauge), ctypes.byref(codec), t0, nt, _ptr(kv_out), _ptr(kv_ref),
        _ptr(err), _stream(stream)))


def cg_cache_error_summary(shape, err_host: np.ndarray) -> dict:
    """err_host float64 [n_fields, 4] -> dict of the whole-cache figures."""
    e = np.ascontiguousarray(err_host, np.float64)
    out = CgCacheError()
    _check("cg_cache_error_summary", lib().cg_cache_error_summary(ctypes.byref(shape), e.ctypes.data,
                                                                  ctypes.byref(out)))
    return {k: getattr(out, k) for k, _ in CgCacheError._fields_}


def cg_adamw_update(param, grad, m, v, step, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                    weight_decay=1e-2):
    """In place on host fp64 arrays of equal size."""
    arrs = [param, grad, m, v]
    for a in arrs:
        assert isinstance(a, np.ndarray) and a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
        assert a.size == param.size
    _check("cg_adamw_update", lib().cg_adamw_update(param.size, *[a.ctypes.data for a in arrs], step,
                                                    lr, beta1, beta2, eps, weight_decay))


def cg_gauge_control(kind, n, g, M=None) -> np.ndarray:
    """-> fp32 [n, g, g] control gauges (M fp64 [n, g, g] for ORTHONORMALIZE / KLT)."""
    G = np.empty((n, g, g), np.float32)
    Mc = np.ascontiguousarray(M, np.float64) if M is not None else None
    if Mc is not None:
        assert Mc.shape == (n, g, g)
    _check("cg_gauge_control", lib().cg_gauge_control(kind, n, g, Mc.ctypes.data if Mc is not None else None,
                                                      G.ctypes.data))
    return G


def cg_second_moment_workspace_bytes(shape, g):
    b = ctypes.c_size_t()
    _check("cg_second_moment_workspace_bytes",
           lib().cg_second_moment_workspace_bytes(ctypes.byref(shape), g, ctypes.byref(b)))
    return b.value


def cg_second_moment(shape, kv, g, workspace, stream=None) -> np.ndarray:
    """-> fp64 [layers, kv, heads, d/g, g, g] second moments (synchronous)."""
    M = np.empty((shape.layers, shape.kv, shape.heads, shape.head_dim // g, g, g), np.float64)
    _check("cg_second_moment", lib().cg_second_moment(ctypes.byref(shape), _ptr(kv), g, _ptr(workspace),
                                                      _nbytes(workspace), M.ctypes.data, _stream(stream)))
    return M


def cg_roundtrip(shape, kv_in, gauge, codec, payload, meta, kv_out, stream=None):
    _check("cg_roundtrip", lib().cg_roundtrip(ctypes.byref(shape), _ptr(kv_in),
                                              ctypes.byref(gauge), ctypes.byref(codec),
                                              _ptr(payload), _nbytes(payload), _ptr(meta),
                                              _nbytes(meta), _ptr(kv_out), _stream(stream)))


def cg_gauge_apply(shape, kv, gauge, direction, out, stream=None):
    _check("cg_gauge_apply", lib().cg_gauge_apply(ctypes.byref(shape), _ptr(kv),
                                                  ctypes.byref(gauge), direction, _ptr(out),
                                                  _stream(stream)))


def cg_gauge_from_skew(A: np.ndarray) -> np.ndarray:
    """A fp64 [n, g, g] (host) -> G = exp(A - A^T) fp32 [n, g, g] (host)."""
    A = np.ascontiguousarray(A, np.float64)
    n, g, _ = A.shape
    G = np.empty((n, g, g), np.float32)
    _check("cg_gauge_from_skew", lib().cg_gauge_from_skew(n, g, A.ctypes.data, G.ctypes.data))
    return G


def cg_gauge_grad(A: np.ndarray, dG: np.ndarray) -> np.ndarray:
    """A, dG fp64 [n, g, g] (host) -> dL/dA fp64 [n, g, g] for G = exp(A - A^T)."""
    A = np.ascontiguousarray(A, np.float64)
    dG = np.ascontiguousarray(dG, np.float64)
    n, g, _ = A.shape
    assert dG.shape == A.shape
    dA = np.empty_like(A)
    _check("cg_gauge_grad", lib().cg_gauge_grad(n, g, A.ctypes.data, dG.ctypes.data, dA.ctypes.data))
    return dA


def cg_stats_workspace_bytes(shape, g, T_b):
    b = ctypes.c_size_t()
    _check("cg_stats_workspace_bytes", lib().cg_stats_workspace_bytes(ctypes.byref(shape), g, T_b,
                                                                      ctypes.byref(b)))
    return b.value


def cg_gauge_fit_stats(shape, kv, g, A_host: np.ndarray, T_b, tau, lambda_f, lambda_r, workspace,
                       grad=True, stream=None):
    """Returns (stats structured array [n_fields], dA fp64 or None)."""
    nf = shape.layers * shape.kv * shape.batch * shape.heads
    out = (CgStats * nf)()
    A = np.ascontiguousarray(A_host, np.float64) if A_host is not None else None
    grad = grad and g != 0
    dA = np.zeros((nf, shape.head_dim // g, g, g), np.float64) if grad else None
    _check("cg_gauge_fit_stats", lib().cg_gauge_fit_stats(
        ctypes.byref(shape), _ptr(kv), g, A.ctypes.data if A is not None else None, T_b, tau,
        lambda_f, lambda_r,
        _ptr(workspace), _nbytes(workspace), ctypes.cast(out, ctypes.c_void_p),
        dA.ctypes.data if grad else None, _stream(stream)))
    stats = np.array([(o.L_freq, o.L_rate, o.L, o.sum_E) for o in out],
                     dtype=[("L_freq", "f8"), ("L_rate", "f8"), ("L", "f8"), ("sum_E", "f8")])
    return stats, dA


def cg_gauge_fit_grad(shape, kv, g, A_host: np.ndarray, T_b, tau, lambda_f, lambda_r, workspace,
                      stream=None):
    """Returns (stats structured array [n_fields], dA fp64 [L, KV, H, D/g, g, g]
    summed over the batch, or None for g = 0)."""
    nf = shape.layers * shape.kv * shape.batch * shape.heads
    out = (CgStats * nf)()
    A = np.ascontiguousarray(A_host, np.float64) if A_host is not None else None
    dA = (np.zeros((shape.layers, shape.kv, shape.heads, shape.head_dim // g, g, g), np.float64)
          if g else None)
    _check("cg_gauge_fit_grad", lib().cg_gauge_fit_grad(
        ctypes.byref(shape), _ptr(kv), g, A.ctypes.data if A is not None else None, T_b, tau,
        lambda_f, lambda_r, _ptr(workspace), _nbytes(workspace), ctypes.cast(out, ctypes.c_void_p),
        dA.ctypes.data if g else None, _stream(stream)))
    stats = np.array([(o.L_freq, o.L_rate, o.L, o.sum_E) for o in out],
                     dtype=[("L_freq", "f8"), ("L_rate", "f8"), ("L", "f8"), ("sum_E", "f8")])
    return stats, dA


def cg_write_header(shape, codec, layer, kv) -> bytes:
    buf = ctypes.create_string_buffer(CG_HEADER_BYTES)
    _check("cg_write_header", lib().cg_write_header(ctypes.byref(shape), ctypes.byref(codec),
                                                    layer, kv, buf, CG_HEADER_BYTES))
    return buf.raw


def cg_last_error() -> str:
    return lib().cg_last_error().decode()
