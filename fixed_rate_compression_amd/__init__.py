"""Codec-Gauge KV-cache round trip on MI355X (gfx950).

The computation lives in the HIP library lib/libcodecgauge.so (C ABI in
include/codec_gauge.h); ``binding`` holds the ctypes marshalling with the
same function names.  Importing this package does not load the library.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    CG_BACKEND_BLOCK_UNIFORM, CG_BACKEND_KIVI, CG_BACKEND_NONE, CG_BACKEND_ZFP, CG_DTYPE_BF16,
    CG_DTYPE_F32, CodecGaugeError, cg_decode, cg_encode, cg_encoded_bytes, cg_gauge_apply,
    cg_gauge_fit_grad, cg_gauge_fit_stats, cg_gauge_from_skew, cg_last_error, cg_roundtrip,
    cg_stats_workspace_bytes, cg_write_header, make_codec, make_gauge, make_shape)
