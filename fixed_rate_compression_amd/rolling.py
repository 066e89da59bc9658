"""Rolling compressed history over the C ABI ("Codec-Gauge", arXiv HTML,
evaluation-protocol paragraph: compressed conditions keep their own
histories, so every new KV token passes through gauge -> backend -> decode ->
inverse gauge).

One history buffer [fields, capacity, 128] (storage format) is the cache the
attention reads.  The model writes each new token's K/V into row t.  When a
4-token block row completes, cg_encode writes its fixed-rate codes at their
fixed stream offset (an append: no other codes move); then cg_decode rewrites
every encoded row [0, 4 floor(t/4)) with its reconstruction.  Rows of the
incomplete block stay as written (at most 3 per field).  All arithmetic runs
in the HIP library; this class only chooses rows and owns buffers.
"""
from __future__ import annotations

from . import binding as cg


class RollingHistory:
    def __init__(self, layers, kv, batch, heads, capacity, gauge, rate, dtype=cg.CG_DTYPE_BF16,
                 head_dim=128):
        import torch

        assert capacity % 4 == 0
        self.dims = (layers, kv, batch, heads)
        self.capacity = capacity
        self.head_dim = head_dim
        self.dtype = dtype
        self.gauge = gauge
        self.codec = cg.make_codec(cg.CG_BACKEND_ZFP, rate)
        self.fields = layers * kv * batch * heads
        tdt = torch.bfloat16 if dtype == cg.CG_DTYPE_BF16 else torch.float32
        self.history = torch.zeros((self.fields, capacity, head_dim), dtype=tdt, device="cuda")
        nbytes = cg.cg_encoded_bytes(self.shape(capacity), self.codec)[0]
        self.payload = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        self.t = 0

    def shape(self, tokens):
        L, KV, B, H = self.dims
        return cg.make_shape(L, KV, B, H, tokens, self.capacity, self.head_dim, self.dtype)

    def prefill(self, kv, T0):
        """Take rows [0, T0) of kv [fields, >=T0, d] as the initial history
        (T0 % 4 == 0): encode them once and decode them."""
        assert T0 % 4 == 0
        self.history[:, :T0].copy_(kv[:, :T0])
        self.t = T0
        sh = self.shape(T0)
        cg.cg_encode(sh, self.history, self.gauge, self.codec, 0, T0, self.payload)
        cg.cg_decode(sh, self.payload, None, self.gauge, self.codec, 0, T0, self.history)

    def append(self, token_kv):
        """One decoding step: token_kv [fields, d] is the new token."""
        t = self.t
        assert t < self.capacity
        self.history[:, t].copy_(token_kv)
        self.t = t + 1
        sh = self.shape(self.t)
        if self.t % 4 == 0:
            cg.cg_encode(sh, self.history, self.gauge, self.codec, self.t - 4, 4, self.payload)
        enc = 4 * (self.t // 4)
        cg.cg_decode(sh, self.payload, None, self.gauge, self.codec, 0, enc, self.history)
