"""cg_decode_error_noalloc (the allocation-free variant of cg_decode_error for
callers that cannot allocate device memory) against cg_decode_error with a
caller workspace: the same kernels, so decoded rows and per-field error sums
must be identical.  Two calls in a row, the second on a smaller input, so the
built-in scratch is reused with stale contents from the first call."""
import numpy as np
import pytest

from fixed_rate_compression_amd import binding as cg
from gpu_util import D, empty_u8, gauges_for, kv_cpu, n_fields, to_dev, to_host

pytestmark = pytest.mark.gpu


def _both(x, G, g, codec, L, KV, B, H, T, bf16):
    t = __import__("torch")
    shape = cg.make_shape(L, KV, B, H, T, T, D, cg.CG_DTYPE_BF16 if bf16 else cg.CG_DTYPE_F32)
    gauge = cg.make_gauge(g, to_dev(np.ascontiguousarray(G)) if G is not None else None)
    xd = to_dev(x)
    pb, mb, _ = cg.cg_encoded_bytes(shape, codec)
    pay = empty_u8(pb)
    meta = t.zeros(max(mb // 4, 1), dtype=t.float32, device="cuda") if mb else None
    cg.cg_encode(shape, xd, gauge, codec, 0, T, pay, meta)
    F = n_fields(L, KV, B, H)
    ws = empty_u8(cg.cg_decode_error_workspace_bytes(shape, gauge, codec, 0, T))
    o1, o2 = t.zeros_like(xd), t.full_like(xd, 7)
    e1 = t.zeros((F, 4), dtype=t.float64, device="cuda")
    e2 = t.full((F, 4), -1.0, dtype=t.float64, device="cuda")
    cg.cg_decode_error(shape, pay, meta, gauge, codec, 0, T, o1, xd, ws, e1)
    cg.cg_decode_error_noalloc(shape, pay, meta, gauge, codec, 0, T, o2, xd, e2)
    t.cuda.synchronize()
    return to_host(o1), to_host(o2), e1.cpu().numpy(), e2.cpu().numpy()


@pytest.mark.parametrize("codec_args,g,bf16", [
    ((cg.CG_BACKEND_ZFP, 4), 16, True),
    ((cg.CG_BACKEND_KIVI, 4, 32, 128), 128, True),
    ((cg.CG_BACKEND_BLOCK_UNIFORM, 3, 64, 0), 8, False),
])
def test_noalloc_matches_workspace_variant_two_calls(codec_args, g, bf16):
    codec = cg.make_codec(*codec_args)
    # first call: 2 layers x K/V x 2 heads x 2112 tokens; second: a smaller cache
    for (L, KV, B, H, T, seed) in ((2, 2, 1, 2, 2112, 900), (1, 2, 1, 1, 448, 901)):
        x = kv_cpu(seed, L, KV, B, H, T, T, 0.95, 4, bf16=bf16)
        G = gauges_for(seed + 10, L, KV, H, g)
        o1, o2, e1, e2 = _both(x, G, g, codec, L, KV, B, H, T, bf16)
        assert np.array_equal(o1, o2), (L, T)
        assert np.array_equal(e1, e2), (L, T)
        assert np.all(e1[:, 3] == T * D) and np.all(e1[:, 1] > 0)

