"""Pins of the oracle's consumer-side gauge (recovery folded into the
downstream projection).

"Codec-Gauge" (arXiv HTML, gauge-parameterization paragraph): the gauge is a
fixed model-side object; some recovery operations can be folded into the
downstream projections, and on the key side this depends on the positional
encoding.  Reading: with the cache kept in gauged coordinates (k' = G k,
v' = G v per channel group, keys cached after RoPE), attention needs
  scores  q . k = (G q) . k'       -> gauge each query after its RoPE
  output  W_o (G^T u) = (W_o G^T) u -> row r of W_o G^T is G applied to row r
with the KV head's gauges for every query head of its group (grouped-query
attention).  The pins compare a decode-attention step computed both ways,
with the explicit recovery written as plain block-diagonal matrix products
(scipy.linalg.block_diag), not with the oracle's gauge routines.
"""
import numpy as np
import pytest
from scipy.linalg import block_diag

import oracle
from fixed_rate_compression_amd import synth

D = 128


def _softmax(s):
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def _attention(q, K, V, Wo, H, q_heads):
    """One decode step: q [q_heads*D], K/V [H][T][D], Wo [dm][q_heads*D] (fp64)."""
    ratio = q_heads // H
    o = np.empty(q_heads * D)
    for h in range(q_heads):
        qh = q[h * D:(h + 1) * D]
        p = _softmax(K[h // ratio] @ qh / np.sqrt(D))
        o[h * D:(h + 1) * D] = p @ V[h // ratio]
    return Wo @ o


def _case(g, seed):
    rng = np.random.default_rng(seed)
    H, q_heads, T, dm = 2, 8, 24, 48
    GK = oracle.gauge_from_skew(synth.gauge_params(seed, H * (D // g), g)).astype(np.float32)
    GV = oracle.gauge_from_skew(synth.gauge_params(seed + 1, H * (D // g), g)).astype(np.float32)
    GK = GK.reshape(H, D // g, g, g)
    GV = GV.reshape(H, D // g, g, g)
    Kg = rng.standard_normal((H, T, D))        # cache rows as decoded, gauged
    Vg = rng.standard_normal((H, T, D))
    q = rng.standard_normal(q_heads * D)
    Wo = rng.standard_normal((dm, q_heads * D)) / np.sqrt(q_heads * D)
    return H, q_heads, GK, GV, Kg, Vg, q, Wo


def _explicit(H, q_heads, GK, GV, Kg, Vg, q, Wo):
    # recovery k = G^T k' per group; as rows: k = k' @ blockdiag(G)
    K = np.stack([Kg[h] @ block_diag(*GK[h].astype(np.float64)) for h in range(H)])
    V = np.stack([Vg[h] @ block_diag(*GV[h].astype(np.float64)) for h in range(H)])
    return _attention(q, K, V, Wo, H, q_heads)


def _folded(H, q_heads, GK, GV, Kg, Vg, q, Wo, g):
    qf = oracle.gauge_heads(q[None, :].astype(np.float32), GK, g, q_heads)[0].astype(np.float64)
    Wf = oracle.gauge_heads(Wo.astype(np.float32), GV, g, q_heads).astype(np.float64)
    return _attention(qf, Kg, Vg, Wf, H, q_heads)


@pytest.mark.parametrize("g", [8, 16, 32, 128])
def test_folded_attention_equals_explicit_recovery(g):
    c = _case(g, 700 + g)
    H, q_heads, GK, GV, Kg, Vg, q, Wo = c
    # the same step with q and W_o rounded to fp32 as the folded side sees them
    y1 = _explicit(H, q_heads, GK, GV, Kg, Vg, q.astype(np.float32).astype(np.float64),
                   Wo.astype(np.float32).astype(np.float64))
    y2 = _folded(*c, g)
    assert np.max(np.abs(y1 - y2)) <= 2e-5 * np.max(np.abs(y1)), np.max(np.abs(y1 - y2))


def test_folding_mistakes_are_detected():
    # a transposed gauge, the wrong kind or the wrong head grouping changes the result
    g = 16
    H, q_heads, GK, GV, Kg, Vg, q, Wo = _case(g, 731)
    q32 = q.astype(np.float32).astype(np.float64)
    W32 = Wo.astype(np.float32).astype(np.float64)
    y1 = _explicit(H, q_heads, GK, GV, Kg, Vg, q32, W32)
    scale = np.max(np.abs(y1))
    bad = [
        (np.swapaxes(GK, -1, -2).copy(), GV),   # G^T on the query
        (GK, np.swapaxes(GV, -1, -2).copy()),   # G^T on W_o
        (GV, GK),                               # keys' and values' gauges swapped
        (GK[::-1].copy(), GV),                  # query head h paired with KV head h % H
    ]
    for GKb, GVb in bad:
        y2 = _folded(H, q_heads, GKb, GVb, Kg, Vg, q, Wo, g)
        assert np.max(np.abs(y1 - y2)) > 1e-2 * scale


def test_gauge_heads_identity_and_segments():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((5, 4 * D)).astype(np.float32)
    assert np.array_equal(oracle.gauge_heads(x, None, 0, 4), x)
    G = oracle.gauge_from_skew(synth.gauge_params(9, 2 * 8, 16)).astype(np.float32).reshape(2, 8, 16, 16)
    y = oracle.gauge_heads(x, G, 16, 4)
    # query heads 0, 1 use KV head 0; 2, 3 use KV head 1; the gauge never mixes heads
    for h in range(4):
        seg = slice(h * D, (h + 1) * D)
        ref = oracle.gauge_forward_f64(x[:, seg], G[h // 2], 16)
        assert np.max(np.abs(y[:, seg] - ref)) <= 1e-5 * np.max(np.abs(ref))
    x2 = x.copy()
    x2[:, D:2 * D] += 1.0
    y2 = oracle.gauge_heads(x2, G, 16, 4)
    assert np.array_equal(np.delete(y2, np.s_[D:2 * D], axis=1), np.delete(y, np.s_[D:2 * D], axis=1))
