"""Measurement kernels (libcgprobe.so); nothing on the codec path uses them.

- Streaming HBM kernels that move bytes in the codec kernels' read : write
  proportions with no other work: the practical memory ceiling the zfp
  kernels are quoted against next to the 8 TB/s peak (stream.hip).
- Instruction-issue probes (issue.hip): the rate of single VALU instruction
  forms (which ones pair up in one issue slot), and whether matrix-core and
  VALU work overlap.  `python3 -m fixed_rate_compression_amd.probe issue`;
  `... probe stream` prints the streaming kernels' rates on a 4.29 GB
  tensor, with the decode-shaped kernel in its store patterns.
- LDS read-pattern probe (lds.hip): matrix-operand reads of a 64-row tile at
  several row pitches and swizzles (`... probe lds`)."""
from __future__ import annotations

import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = [os.path.join(_HERE, "stream.hip"), os.path.join(_HERE, "issue.hip"), os.path.join(_HERE, "lds.hip")]
_LIB = os.path.join(_HERE, "libcgprobe.so")

MODES = {"copy": (0, 1, 1), "enc": (1, 4, 1), "dec": (2, 1, 4), "dec_rows": (3, 1, 4), "dec_rows_nt": (4, 1, 4),
         "dec_rows128": (5, 1, 4)}   # name: (mode, read, write)


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "hipcc", "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-o", tmp, *_SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (bind to torch's HIP runtime first)
        if not os.path.exists(_LIB):
            raise RuntimeError("libcgprobe.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB)
        L.cgprobe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                     ctypes.c_uint64, ctypes.c_void_p]
        L.cgprobe_stream.restype = ctypes.c_int
        for fn in (L.cgprobe_issue, L.cgprobe_overlap, L.cgprobe_lds):
            fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.POINTER(ctypes.c_float)]
            fn.restype = ctypes.c_int
        _lib = L
    return _lib


def stream(name: str, src, dst, stream=None) -> None:
    """Launch the `name` kernel ('copy', 'enc', 'dec') over all of src (torch
    device tensors; dst sized for the mode's write share)."""
    import torch
    mode, rin, rout = MODES[name]
    nb = src.numel() * src.element_size()
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    rc = lib().cgprobe_stream(mode, src.data_ptr(), nb, dst.data_ptr(),
                              dst.numel() * dst.element_size(), s)
    if rc != 0:
        raise RuntimeError(f"cgprobe_stream({name}) failed with {rc}")


def ceilings(kv, steps: int = 10, warmup: int = 2, names=("copy", "enc", "dec")) -> dict:
    """HBM GB/s (bytes read + written per second, median over `steps` timed
    launches) of the kernels `names` (keys of MODES) on the tensor `kv` (the
    copy and the encode-shaped kernel read it; the decode-shaped kernels
    read a quarter of its size and write its full size)."""
    import numpy as np
    import torch
    nb = kv.numel() * kv.element_size()
    flat = kv.view(torch.uint8).view(-1)
    out = {}
    for name in names:
        _, rin, rout = MODES[name]
        if rout > rin:
            src = flat[: nb // 4]
            dst = torch.empty(nb, dtype=torch.uint8, device=kv.device)
        else:
            src = flat
            dst = torch.empty(nb * rout // rin, dtype=torch.uint8, device=kv.device)
        moved = src.numel() + dst.numel()
        for _ in range(warmup):
            stream(name, src, dst)
        torch.cuda.synchronize()
        ts = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            stream(name, src, dst)
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        t = float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e-3
        out[name] = {"GBs": round(moved / t / 1e9, 1), "ms": round(t * 1e3, 4), "bytes": moved}
        del dst
        torch.cuda.empty_cache()
    return out


# the instruction forms of issue.hip, in its kernel order
ISSUE_FORMS = ("v_xor_b32, VGPR operands", "v_xor_b32, an SGPR operand", "v_xor_b32, a literal",
               "v_add_u32", "v_bitop3_b32, VGPR operands", "v_bitop3_b32, an SGPR operand",
               "v_lshrrev_b32 by 1", "v_lshlrev_b32 by 1", "v_bfe_u32", "v_perm_b32", "v_lshl_or_b32",
               "v_bcnt_u32_b32", "v_ffbh_u32", "v_min_u32", "v_fma_f32, VGPR operands",
               "v_fma_f32, an SGPR operand", "v_cvt_f32_i32")
OVERLAP_MODES = ("fp32 16x16x4 alone", "VALU alone (fp32 case)", "fp32 16x16x4 + VALU in one wave",
                 "fp32 16x16x4 and VALU in separate waves", "bf16 16x16x32 alone", "VALU alone (bf16 case)",
                 "bf16 16x16x32 + VALU in one wave", "bf16 16x16x32 and VALU in separate waves")


def issue_rates(iters: int = 2000) -> dict:
    """G wave64 instructions/s of each form of ISSUE_FORMS (2048 x 256 threads,
    32 instructions per trip)."""
    import torch
    L = lib()
    assert L.cgprobe_issue_kinds() == len(ISSUE_FORMS)
    out = torch.empty(2048 * 256, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    res = {}
    for k, name in enumerate(ISSUE_FORMS):
        ms = ctypes.c_float()
        if L.cgprobe_issue(k, iters, out.data_ptr(), s, ctypes.byref(ms)) != 0:
            raise RuntimeError(f"cgprobe_issue({k}) failed")
        res[name] = round(2048 * 4 * iters * 32 / (ms.value * 1e-3) / 1e9, 1)
    return res


def overlap_times(iters: int = 2000) -> dict:
    """ms of each mode of OVERLAP_MODES."""
    import torch
    L = lib()
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    res = {}
    for m, name in enumerate(OVERLAP_MODES):
        ms = ctypes.c_float()
        if L.cgprobe_overlap(m, iters, out.data_ptr(), s, ctypes.byref(ms)) != 0:
            raise RuntimeError(f"cgprobe_overlap({m}) failed")
        res[name] = round(ms.value, 3)
    return res


# the read patterns of lds.hip, in its kernel order
LDS_KINDS = ("pitch 68 dwords", "pitch 76 dwords", "pitch 72 dwords", "pitch 64, chunk ^ (row % 8)",
             "pitch 64", "pitch 64, chunk ^ ((row / 2) % 8)")


def lds_times(iters: int = 2000) -> dict:
    """ms of each LDS read pattern of LDS_KINDS (16 ds_read_b128 per trip)."""
    import torch
    L = lib()
    out = torch.empty(2048 * 256, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    res = {}
    for k, name in enumerate(LDS_KINDS):
        ms = ctypes.c_float()
        if L.cgprobe_lds(k, iters, out.data_ptr(), s, ctypes.byref(ms)) != 0:
            raise RuntimeError(f"cgprobe_lds({k}) failed")
        res[name] = round(ms.value, 3)
    return res
