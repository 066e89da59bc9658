"""Gauge training on the frequency objective, the coordinate controls, and
their evaluation ("Codec-Gauge: Learning Compression-Friendly Gauges for
Transformer KV Caches", arXiv HTML: gauge-training paragraph -- AdamW for a
number of epochs over windows of cached KV; main-grid and coordinate-control
paragraphs -- identity, random orthogonal, Hadamard, DCT and PCA/KLT gauges
with the learned gauge's block structure; spectral concentration is tracked as
1 - L_freq).

Orchestration only: the statistics and their gradient, the AdamW update, the
control gauges, the second moments and the codec round trips are calls into
libcodecgauge.so.  Windows are 4096-token row ranges of one [fields][rows][128]
device tensor; a training step takes one window, and the gradient of the
objective summed over the fields that share a gauge (the batch) updates that
gauge's skew parameters A, starting from A = 0 (identity coordinates).
"""
from __future__ import annotations

import numpy as np

from . import binding as cg


def _window(x, w, Tw):
    """raw device address of rows [w Tw, (w+1) Tw) of every field of x [F, rows, D]"""
    return x.data_ptr() + w * Tw * x.shape[2] * x.element_size()


def _dtype(x):
    import torch
    return cg.CG_DTYPE_BF16 if x.dtype == torch.bfloat16 else cg.CG_DTYPE_F32


def control_gauges(kind: str, L, KV, H, g, D=128, seed=0, moments=None) -> np.ndarray:
    """fp32 [L, KV, H, D/g, g, g] gauges of one condition: 'identity',
    'hadamard', 'dct', 'random' (Haar, from seeded Gaussian matrices) or
    'klt' (moments: fp64 [L, KV, H, D/g, g, g] from second_moments())."""
    n = L * KV * H * (D // g)
    if kind == "identity":
        G = cg.cg_gauge_control(cg.CG_CONTROL_IDENTITY, n, g)
    elif kind == "hadamard":
        G = cg.cg_gauge_control(cg.CG_CONTROL_HADAMARD, n, g)
    elif kind == "dct":
        G = cg.cg_gauge_control(cg.CG_CONTROL_DCT, n, g)
    elif kind == "random":
        M = np.random.default_rng(seed).standard_normal((n, g, g))
        G = cg.cg_gauge_control(cg.CG_CONTROL_ORTHONORMALIZE, n, g, M)
    elif kind == "klt":
        G = cg.cg_gauge_control(cg.CG_CONTROL_KLT, n, g, np.asarray(moments).reshape(n, g, g))
    else:
        raise ValueError(kind)
    return G.reshape(L, KV, H, D // g, g, g)


def second_moments(x, L, KV, B, H, g, tokens=None):
    """Per-gauge uncentered second moments of x [F, rows, 128] over rows [0, tokens)."""
    import torch
    T = x.shape[1] if tokens is None else tokens
    shape = cg.make_shape(L, KV, B, H, T, x.shape[1], x.shape[2], _dtype(x))
    ws = torch.empty(cg.cg_second_moment_workspace_bytes(shape, g), dtype=torch.uint8, device=x.device)
    return cg.cg_second_moment(shape, x, g, ws)


class GaugeTrainer:
    """AdamW on A (fp64 [L, KV, H, D/g, g, g]) over the windows of x."""

    def __init__(self, x, L, KV, B, H, g, window=4096, lr=1e-3, betas=(0.9, 0.999), eps=1e-8,
                 weight_decay=1e-2, T_b=16, tau=0.04, lambda_f=1.0, lambda_r=0.02):
        import torch
        self.x, self.L, self.KV, self.B, self.H, self.g = x, L, KV, B, H, g
        self.D = x.shape[2]
        self.Tw = window
        self.W = x.shape[1] // window
        assert self.W >= 1 and x.is_contiguous()
        self.hyper = dict(lr=lr, beta1=betas[0], beta2=betas[1], eps=eps, weight_decay=weight_decay)
        self.obj = dict(T_b=T_b, tau=tau, lambda_f=lambda_f, lambda_r=lambda_r)
        self.A = np.zeros((L, KV, H, self.D // g, g, g))
        self.m = np.zeros_like(self.A)
        self.v = np.zeros_like(self.A)
        self.t = 0
        self.shape = cg.make_shape(L, KV, B, H, window, x.shape[1], self.D, _dtype(x))
        self.ws = torch.empty(cg.cg_stats_workspace_bytes(self.shape, g, T_b), dtype=torch.uint8,
                              device=x.device)
        self.history = []

    def step(self, w: int) -> float:
        """One AdamW step on window w; returns the mean objective L before it."""
        o = self.obj
        # fields (l, s, b, h) share the gauge (l, s, h): the library returns the
        # gradient of the batch objective per gauge
        st, grad = cg.cg_gauge_fit_grad(self.shape, _window(self.x, w, self.Tw), self.g, self.A,
                                         o["T_b"], o["tau"], o["lambda_f"], o["lambda_r"], self.ws)
        self.t += 1
        flat = [np.ascontiguousarray(a).reshape(-1) for a in (self.A, grad, self.m, self.v)]
        cg.cg_adamw_update(flat[0], flat[1], flat[2], flat[3], self.t, **self.hyper)
        self.A, self.m, self.v = (flat[0].reshape(self.A.shape), flat[2].reshape(self.A.shape),
                                  flat[3].reshape(self.A.shape))
        loss = float(np.mean(st["L"]))
        self.history.append(loss)
        return loss

    def fit(self, epochs: int):
        for _ in range(epochs):
            for w in range(self.W):
                self.step(w)
        return self.A

    def gauges(self) -> np.ndarray:
        """fp32 G = exp(A - A^T) of the current parameters."""
        g = self.g
        return cg.cg_gauge_from_skew(self.A.reshape(-1, g, g)).reshape(self.A.shape).astype(np.float32)

    def save(self, path):
        """Checkpoint of the training state (parameters, AdamW moments, step
        count, settings, loss history) as an .npz file (no pickled objects)."""
        np.savez(path, A=self.A, m=self.m, v=self.v, t=np.int64(self.t), g=np.int32(self.g),
                 window=np.int64(self.Tw), history=np.asarray(self.history, np.float64),
                 hyper=np.array([self.hyper[k] for k in _HYPER], np.float64),
                 obj=np.array([self.obj[k] for k in _OBJ], np.float64))

    def load(self, path):
        """Resume from save(): the same cache shape, group and window are required."""
        with np.load(path, allow_pickle=False) as z:
            if int(z["g"]) != self.g or int(z["window"]) != self.Tw or z["A"].shape != self.A.shape:
                raise ValueError("checkpoint does not match this trainer's shape, group or window")
            self.A, self.m, self.v = (np.array(z[k], np.float64) for k in ("A", "m", "v"))
            self.t = int(z["t"])
            self.history = [float(h) for h in z["history"]]
            self.hyper = dict(zip(_HYPER, (float(h) for h in z["hyper"])))
            self.obj = dict(zip(_OBJ, (float(o) for o in z["obj"])))
            self.obj["T_b"] = int(self.obj["T_b"])
        return self


_HYPER = ("lr", "beta1", "beta2", "eps", "weight_decay")
_OBJ = ("T_b", "tau", "lambda_f", "lambda_r")


def save_gauges(path, A: np.ndarray, g: int):
    """A gauge set as a model-side file: the skew parameters A (fp64) and the
    fp32 gauges G = exp(A - A^T) the kernels use, [L, KV, H, D/g, g, g] each."""
    A = np.asarray(A, np.float64)
    G = cg.cg_gauge_from_skew(A.reshape(-1, g, g)).reshape(A.shape).astype(np.float32)
    np.savez(path, A=A, G=G, g=np.int32(g))


def load_gauges(path):
    """-> (A fp64, G fp32, g) from save_gauges; G is checked against exp(A - A^T)."""
    with np.load(path, allow_pickle=False) as z:
        A, G, g = np.array(z["A"], np.float64), np.array(z["G"], np.float32), int(z["g"])
    if A.shape != G.shape or A.shape[-2:] != (g, g):
        raise ValueError("gauge file: A and G shapes do not match the group size")
    G_ref = cg.cg_gauge_from_skew(A.reshape(-1, g, g)).reshape(A.shape).astype(np.float32)
    if not np.array_equal(G.view(np.uint32), G_ref.view(np.uint32)):
        raise ValueError("gauge file: G is not exp(A - A^T) of the stored A")
    return A, G, g


def evaluate(x, L, KV, B, H, g, G, rates=(3, 4, 6), T_b=16, tau=0.04, lambda_f=1.0, lambda_r=0.02):
    """Spectral concentration 1 - L_freq of the gauged cache and the zfp-style
    round-trip error at each rate, for gauges G fp32 [L, KV, H, D/g, g, g]
    (None = identity).  x [F, T, 128] on the device."""
    import torch
    F, T, D = x.shape
    dt = _dtype(x)
    shape = cg.make_shape(L, KV, B, H, T, T, D, dt)
    Gd = torch.from_numpy(np.ascontiguousarray(G, np.float32)).to(x.device) if G is not None else None
    gauge = cg.make_gauge(g if G is not None else 0, Gd)
    # statistics of the gauged cache: apply the gauge, then the identity-gauge statistics
    xg = torch.empty((F, T, D), dtype=torch.float32, device=x.device)
    cg.cg_gauge_apply(shape, x, gauge, 0, xg)         # (g = 0: plain widening copy)
    s32 = cg.make_shape(L, KV, B, H, T, T, D, cg.CG_DTYPE_F32)
    ws = torch.empty(cg.cg_stats_workspace_bytes(s32, 0, T_b), dtype=torch.uint8, device=x.device)
    st, _ = cg.cg_gauge_fit_stats(s32, xg, 0, None, T_b, tau, lambda_f, lambda_r, ws, grad=False)
    del xg
    res = {"spectral_concentration": float(1.0 - np.mean(st["L_freq"])), "L": float(np.mean(st["L"]))}
    out = torch.empty_like(x)
    err = torch.empty((F, 4), dtype=torch.float64, device=x.device)
    for R in rates:
        codec = cg.make_codec(cg.CG_BACKEND_ZFP, R)
        pb, _, _ = cg.cg_encoded_bytes(shape, codec)
        pay = torch.empty(pb, dtype=torch.uint8, device=x.device)
        wse = torch.empty(max(cg.cg_decode_error_workspace_bytes(shape, gauge, codec, 0, T), 8),
                          dtype=torch.uint8, device=x.device)
        cg.cg_encode(shape, x, gauge, codec, 0, T, pay)
        cg.cg_decode_error(shape, pay, None, gauge, codec, 0, T, out, x, wse, err)
        summ = cg.cg_cache_error_summary(shape, err.cpu().numpy())
        res[f"zfp{R}_nrmse"] = summ["nrmse"]
        res[f"zfp{R}_key_nrmse"] = summ["key_nrmse"]
        res[f"zfp{R}_value_nrmse"] = summ["value_nrmse"]
    return res
