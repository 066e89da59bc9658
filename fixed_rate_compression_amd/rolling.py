"""Rolling compressed history over the C ABI ("Codec-Gauge", arXiv HTML,
evaluation-protocol paragraph: compressed conditions keep their own
histories, so every new KV token passes through gauge -> backend -> decode ->
inverse gauge).

One history buffer [fields, capacity, 128] (storage format) is the cache the
attention reads.  The model writes each new token's K/V into row t.

every_token=True (default; the protocol above): after each append the 4-token
block row that holds the new token is encoded from its raw tokens (a partial
block row is padded by repeating its last token; a small side buffer keeps the
raw tokens of the current block row, since the history rows hold
reconstructions), its codes overwrite that block row's fixed stream offset,
and cg_decode rewrites every row [0, t+1) with its reconstruction.

every_token=False: only completed block rows are encoded and decoded; the at
most 3 rows of the incomplete block stay as written.

keep (CG_KEEP_KEYS | CG_KEEP_VALUES, every-token mode only): the history
holds those kinds in gauged coordinates (cg_decode_gauged), for a consumer
that folds the recovery into its query and output projection
(cg_gauge_heads).

All arithmetic runs in the HIP library; this class only chooses rows and owns
buffers.
"""
from __future__ import annotations

from . import binding as cg


class RollingHistory:
    def __init__(self, layers, kv, batch, heads, capacity, gauge, rate, dtype=cg.CG_DTYPE_BF16,
                 head_dim=128, every_token=True, keep=0):
        import torch

        assert capacity % 4 == 0
        self.dims = (layers, kv, batch, heads)
        self.capacity = capacity
        self.head_dim = head_dim
        self.dtype = dtype
        self.gauge = gauge
        self.every_token = every_token
        assert every_token or not keep, "a gauged history needs every-token mode"
        self.keep = keep
        self.codec = cg.make_codec(cg.CG_BACKEND_ZFP, rate)
        self.fields = layers * kv * batch * heads
        tdt = torch.bfloat16 if dtype == cg.CG_DTYPE_BF16 else torch.float32
        self.history = torch.zeros((self.fields, capacity, head_dim), dtype=tdt, device="cuda")
        self.raw_row = torch.zeros((self.fields, 4, head_dim), dtype=tdt, device="cuda")
        nbytes = cg.cg_encoded_bytes(self.shape(capacity), self.codec)[0]
        self.payload = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        self.t = 0

    def shape(self, tokens):
        L, KV, B, H = self.dims
        return cg.make_shape(L, KV, B, H, tokens, self.capacity, self.head_dim, self.dtype)

    def _decode(self, sh, n):
        cg.cg_decode_gauged(sh, self.payload, None, self.gauge, self.codec, 0, n, self.keep,
                            self.history)

    def prefill(self, kv, T0):
        """Take rows [0, T0) of kv [fields, >=T0, d] as the initial history:
        encode them once and decode them (completed-block mode: the rows of a
        partial last block row stay raw)."""
        self.history[:, :T0].copy_(kv[:, :T0])
        b = 4 * (T0 // 4)
        self.raw_row[:, :T0 - b].copy_(kv[:, b:T0])
        self.t = T0
        sh = self.shape(T0)
        n = T0 if self.every_token else b
        if n:
            cg.cg_encode(sh, self.history, self.gauge, self.codec, 0, n, self.payload)
            self._decode(sh, n)

    def append(self, token_kv):
        """One decoding step: token_kv [fields, d] is the new token."""
        t = self.t
        assert t < self.capacity
        self.t = t + 1
        sh = self.shape(self.t)
        b = 4 * (t // 4)
        if self.every_token:
            # the block row [b, t+1) from its raw tokens, padded when partial
            self.raw_row[:, t - b].copy_(token_kv)
            self.history[:, b:t + 1].copy_(self.raw_row[:, :t + 1 - b])
            cg.cg_encode(sh, self.history, self.gauge, self.codec, b, t + 1 - b, self.payload)
            self._decode(sh, self.t)
            return
        self.raw_row[:, t - b].copy_(token_kv)
        self.history[:, t].copy_(token_kv)
        if self.t % 4 == 0:
            cg.cg_encode(sh, self.history, self.gauge, self.codec, self.t - 4, 4, self.payload)
        enc = 4 * (self.t // 4)
        cg.cg_decode(sh, self.payload, None, self.gauge, self.codec, 0, enc, self.history)

    # ------------------------------------------------------------------
    # checkpoint / resume: the fixed-rate stream, the raw tokens of the
    # current block row and the token count are the whole state; the history
    # is rebuilt by decoding
    # ------------------------------------------------------------------
    def save(self, path):
        """Write the history's state to an .npz file (no pickled objects)."""
        import numpy as np
        import torch
        torch.cuda.synchronize()
        raw = self.raw_row.cpu()
        if raw.dtype == torch.bfloat16:
            raw = raw.view(torch.int16)
        np.savez(path, payload=self.payload.cpu().numpy(), raw_row=raw.numpy(), t=np.int64(self.t),
                 dims=np.array(self.dims, np.int64), capacity=np.int64(self.capacity),
                 rate=np.int32(self.codec.bits), dtype=np.int32(self.dtype),
                 head_dim=np.int32(self.head_dim), every_token=np.int32(self.every_token),
                 keep=np.int32(self.keep))

    @classmethod
    def restore(cls, path, gauge):
        """Rebuild a history saved by save(); `gauge` is the model-side gauge
        set it was built with (not part of the state)."""
        import numpy as np
        import torch
        with np.load(path, allow_pickle=False) as z:
            L, KV, B, H = (int(v) for v in z["dims"])
            rh = cls(L, KV, B, H, int(z["capacity"]), gauge, int(z["rate"]), int(z["dtype"]),
                     int(z["head_dim"]), bool(z["every_token"]), int(z["keep"]))
            payload, raw, t = z["payload"], z["raw_row"], int(z["t"])
        if payload.size != rh.payload.numel() or raw.shape != tuple(rh.raw_row.shape):
            raise ValueError("saved state does not match the history's shape")
        rh.payload.copy_(torch.from_numpy(payload))
        raw_t = torch.from_numpy(raw)
        rh.raw_row.copy_(raw_t.view(torch.bfloat16) if rh.raw_row.dtype == torch.bfloat16 else raw_t)
        rh.t = t
        if t:
            b = 4 * (t // 4)
            if rh.every_token:
                rh._decode(rh.shape(t), t)
            else:
                if b:
                    cg.cg_decode(rh.shape(t), rh.payload, None, rh.gauge, rh.codec, 0, b, rh.history)
                rh.history[:, b:t].copy_(rh.raw_row[:, :t - b])
        return rh
