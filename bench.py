"""Benchmark: KV GB/s of the fused gauge + encode and decode + inverse-gauge
kernels at 4 bits/value, and their fraction of MI355X HBM bandwidth.

Workload (one GPU): a Llama-3-8B-class GQA cache, 32 layers x K/V x 8 KV
heads x head_dim 128 x 32768 tokens, bf16 storage, synthetic values
(lognormal channel scales, AR(1) rho = 0.95 along tokens, 4 outlier channels
at 20x per head), gauge g = 16 from A ~ N(0, 0.1^2), zfp-style fixed rate
4 bits/value.  One step = gauge + encode of the whole cache followed by
decode + inverse gauge of the whole cache; inputs are resident in HBM.

Prints one JSON line: the metric, value (round-trip KV GB/s), timing
(medians of HIP-event times), the configuration, per-direction figures, the
roofline object of the slower kernel (algorithmic bytes per launch over its
HIP-event time, against the 8 TB/s HBM peak and against the streaming-kernel
ceiling measured in the same run; the rocprofv3-measured HBM traffic and
VALU instruction count when the kernel sources match the ones the counters
were taken on, with the instruction rate against the chip's single-issue
VALU rate; `bound` names the resource with the larger measured fraction),
the CPU oracle baseline on a bounded sample, and `configs`: the encode and
decode figures of every other workload (small fp32 cache, the other zfp
rates, the full-head gauge quantizers, the rolling history, the 27B-class
cache and its gauge-fit statistics), measured in the same run.
--workload selects the detailed lines of one workload, one JSON line each.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV GB/s for gauge+encode and decode+inverse at 4 bits/value; % of HBM peak"
HBM_PEAK_GBS = 8000.0
# Instruction-issue slots of the chip: a SIMD issues one wave64 VALU
# instruction per 4 cycles, so 256 CUs x 4 SIMDs x 2.4 GHz / 4 = 614.4 G
# slots/s.  Two instructions of different waves share a slot when both are
# eligible for dual issue (simple 32-bit logic, add/sub, right shifts, fp32
# add/mul/fma with VGPR or literal operands, measured on gfx950; counted by
# SQ_ACTIVE_INST_VALU2), and a matrix instruction holds its SIMD for its
# cycles except those in which VALU work co-executes (bf16 forms do, the
# fp32 16x16x4 form does not).  Slots used per launch = VALU instructions -
# dual-issued pairs + (matrix busy - co-executed cycles) / 4.
ISSUE_SLOTS_PEAK_GPS = 256 * 4 * 2.4 / 4

# HBM bytes per launch of the fused zfp kernels on this workload, from two
# rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) scaled by what the same
# counters read for a plain device copy of the KV tensor (fetch x 2.0, write
# x 1.0).  They hold only for the kernel sources they were taken on: bench.py
# reports null once the hash of those sources differs.
PMC_SOURCES = ("cg_launch.hpp", "cg_tile.hpp", "gauge128.hpp", "split_gauge.hpp", "zfp_block.hpp",
               "zfp_kernels.hpp", "zfp_r4.hip", "kernels_zfp.hip", "../build.py")
PMC_TRAFFIC = {"sha256": "9f8302f9bb9e1c6b5e30de7f1f08e219f0024d257bf2d4b2079f27e162212882",
               # FETCH_SIZE x 2 + WRITE_SIZE x 1 (KiB -> B), per launch
               "k_zfp_encode": 5402689621, "k_zfp_decode": 5406598272,
               # per launch (rocprofv3 --pmc, same sources): SQ_INSTS_VALU,
               # SQ_ACTIVE_INST_VALU2, SQ_VALU_MFMA_BUSY_CYCLES, SQ_VALU_MFMA_COEXEC_CYCLES
               "valu_k_zfp_encode": 1204511363, "valu2_k_zfp_encode": 182045782,
               "mfma_k_zfp_encode": 1073741824, "coexec_k_zfp_encode": 0,
               "valu_k_zfp_decode": 1373576982, "valu2_k_zfp_decode": 280576980,
               "mfma_k_zfp_decode": 335495456, "coexec_k_zfp_decode": 173685605}

CFG = dict(layers=32, kv=2, batch=1, heads=8, tokens=32768, head_dim=128, g=16, rate=4,
           rho=0.95, outliers=4, seed=2)


def kernel_sources_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in PMC_SOURCES:
        with open(os.path.join(ROOT, "fixed_rate_compression_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    return PMC_TRAFFIC.get(kernel) if kernel_sources_sha() == PMC_TRAFFIC["sha256"] else None


def issue_slots(kernel: str, seconds: float):
    """The kernel's instruction-issue figures per launch from the counters
    (null when the sources changed since they were taken): slots used and
    their rate against ISSUE_SLOTS_PEAK_GPS."""
    v, v2, mb, co = (measured_traffic(k + "_" + kernel) for k in ("valu", "valu2", "mfma", "coexec"))
    if v is None:
        return {"issue_slots_per_launch": None, "achieved": None, "peak": ISSUE_SLOTS_PEAK_GPS,
                "unit": "G SIMD issue slots/s", "frac": None}
    slots = v - v2 + (mb - co) / 4
    gps = slots / seconds / 1e9
    return {"issue_slots_per_launch": int(slots), "achieved": round(gps, 1), "peak": ISSUE_SLOTS_PEAK_GPS,
            "unit": "G SIMD issue slots/s", "frac": round(gps / ISSUE_SLOTS_PEAK_GPS, 4),
            "valu_instr_per_launch": v, "dual_issued_pairs": v2,
            "matrix_cycles_not_coexecuted": mb - co}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def setup(rate=None):
    import torch

    from fixed_rate_compression_amd import binding as cg
    from fixed_rate_compression_amd import synth

    c = CFG
    L, KV, B, H, T, D, g = c["layers"], c["kv"], c["batch"], c["heads"], c["tokens"], c["head_dim"], c["g"]
    R = rate or c["rate"]
    F = L * KV * B * H
    x = torch.empty((F, T, D), dtype=torch.bfloat16, device="cuda")
    synth.generate_gpu(x, T, c["rho"], c["seed"], np.arange(F),
                       synth.channel_scales_many(c["seed"], range(F), D, c["outliers"]))
    A = synth.gauge_params(c["seed"] + 100, L * KV * H * (D // g), g)
    G = torch.from_numpy(cg.cg_gauge_from_skew(A)).cuda()
    shape = cg.make_shape(L, KV, B, H, T, T, D, cg.CG_DTYPE_BF16)
    codec = cg.make_codec(cg.CG_BACKEND_ZFP, R)
    gauge = cg.make_gauge(g, G)
    pbytes, mbytes, hbytes = cg.cg_encoded_bytes(shape, codec)
    pay = torch.empty(pbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    torch.cuda.synchronize()
    return dict(x=x, G=G, A=A, shape=shape, codec=codec, gauge=gauge, pay=pay, out=out,
                pbytes=pbytes, hbytes=hbytes, N=F * T * D, F=F, T=T, D=D, R=R, g=g)


def step(s, ev=None):
    from fixed_rate_compression_amd import binding as cg
    if ev is not None:
        ev[0].record()
    cg.cg_encode(s["shape"], s["x"], s["gauge"], s["codec"], 0, s["T"], s["pay"])
    if ev is not None:
        ev[1].record()
    cg.cg_decode(s["shape"], s["pay"], None, s["gauge"], s["codec"], 0, s["T"], s["out"])
    if ev is not None:
        ev[2].record()


def time_steps(s, steps, warmup):
    import torch
    for _ in range(warmup):
        step(s)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(s, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    dec = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    return wall, enc, dec


def host_threads() -> int:
    """Worker threads for the CPU baseline: the cores this process may run on,
    at most 16 (a one-GPU machine's CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(s):
    """The oracle (plain C + numpy, untuned) on a bounded sample of the same
    workload: every field of layers 0, L/2 and L-1 (K and V, all heads), a
    full round trip (gauge, encode, decode, inverse gauge) per field, one
    field per worker thread; the rate and a labelled extrapolation of the
    whole cache's time at that rate."""
    import concurrent.futures as cf

    import torch

    import oracle
    x = s["x"]
    D, T, R, g = s["D"], s["T"], s["R"], s["g"]
    L, KV, H = CFG["layers"], CFG["kv"], CFG["heads"]
    Gh = s["G"].cpu().numpy().reshape(L, KV, H, D // g, g, g)
    layers = sorted({0, L // 2, L - 1})
    fields = [(l * KV + kv) * H + h for l in layers for kv in range(KV) for h in range(H)]
    host = [x[f].view(torch.int16).cpu().numpy().view(np.uint16) for f in fields]
    threads = min(host_threads(), len(fields))

    def one(i):
        f = fields[i]
        h, ls = f % H, f // H
        oracle.zfp_roundtrip_field(host[i], Gh[ls // KV, ls % KV, h], g, R)

    oracle.lib()
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(len(fields))))
    wall = time.perf_counter() - t0
    nvals = len(fields) * T * D
    rate = nvals * 2 / wall / 1e9
    return dict(value=round(rate, 4), unit="GB/s", cores=threads, kind="oracle",
                sample=f"all {len(fields)} fields of layers {layers} ({nvals} values, "
                       f"{len(fields)} of {s['F']} fields), gauge+encode+decode+inverse round trip, "
                       f"{wall:.2f} s wall on {threads} threads",
                extrapolated_full_cache_s=round(s["N"] * 2 / 1e9 / rate, 2),
                extrapolation="labelled estimate: the whole cache's round trip at the sampled rate "
                              "(fields are independent and equal in size)")


# ---------------------------------------------------------------------------
# the other workloads (one JSON line each with --workload all)
# ---------------------------------------------------------------------------

def _gen(F, T, Tcap, rho, seed, outliers, bf16, scale_seed=None, windows=1):
    """Synthetic cache: per-field channel scales from scale_seed (default: seed),
    token noise from seed -- equal scale seeds give the same 'model' with
    different text."""
    import torch

    from fixed_rate_compression_amd import synth
    D = 128
    x = torch.zeros((F * windows, Tcap // windows, D), dtype=torch.bfloat16 if bf16 else torch.float32,
                    device="cuda")
    sc = synth.channel_scales_many(seed if scale_seed is None else scale_seed, range(F), D, outliers)
    if windows > 1:
        sc = np.repeat(sc, windows, axis=0)
    synth.generate_gpu(x, T // windows, rho, seed, np.arange(F * windows), sc)
    return x.view(F, Tcap, D)


def _gauge(L, KV, H, g, seed):
    import torch

    from fixed_rate_compression_amd import binding as cg
    from fixed_rate_compression_amd import synth
    if g == 0:
        return None, None
    A = synth.gauge_params(seed, L * KV * H * (128 // g), g)
    return torch.from_numpy(cg.cg_gauge_from_skew(A)).cuda(), A


def _time(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e-3


def _codec_line(name, shape, x, G, g, codec, steps, warmup, esz, desc, folded=True):
    import torch

    from fixed_rate_compression_amd import binding as cg
    pb, mb, hb = cg.cg_encoded_bytes(shape, codec)
    pay = torch.empty(max(pb, 1), dtype=torch.uint8, device="cuda")
    meta = torch.empty(max(mb // 4, 1), dtype=torch.float32, device="cuda") if mb else None
    out = torch.empty_like(x)
    gauge = cg.make_gauge(g, G)
    T = shape.tokens
    enc = lambda: cg.cg_encode(shape, x, gauge, codec, 0, T, pay, meta)
    dec = lambda: cg.cg_decode(shape, pay, meta, gauge, codec, 0, T, out)
    enc()
    te = _time(enc, steps, warmup)
    td = _time(dec, steps, warmup)
    # decode with the cache-side error sums against the input (fused in the decode kernels)
    ws = torch.empty(max(cg.cg_decode_error_workspace_bytes(shape, gauge, codec, 0, T), 8),
                     dtype=torch.uint8, device="cuda")
    err = torch.empty((x.shape[0], 4), dtype=torch.float64, device="cuda")
    dece = lambda: cg.cg_decode_error(shape, pay, meta, gauge, codec, 0, T, out, x, ws, err)
    tde = _time(dece, steps, warmup)
    summ = cg.cg_cache_error_summary(shape, err.cpu().numpy())
    # recovery folded into the consumer: values (or keys and values) left gauged
    fold = {}
    if g and folded:
        for nm, keep in (("values", cg.CG_KEEP_VALUES), ("both", cg.CG_KEEP_KEYS | cg.CG_KEEP_VALUES)):
            fn = lambda keep=keep: cg.cg_decode_gauged(shape, pay, meta, gauge, codec, 0, T, keep, out)
            fold[f"decode_folded_{nm}_ms"] = round(_time(fn, steps, warmup) * 1e3, 4)
    N = x.numel()
    alg = N * esz + pb + mb
    del pay, meta, out, ws
    torch.cuda.empty_cache()
    return {"workload": name, "desc": desc, "values": N, "bits_per_value": round(8.0 * (pb + mb + hb) / N, 6),
            "kv_nrmse": round(summ["nrmse"], 6), "key_nrmse": round(summ["key_nrmse"], 6),
            "value_nrmse": round(summ["value_nrmse"], 6), "kv_mse": summ["mse"],
            "max_abs_err": summ["max_abs"], "decode_with_error_ms": round(tde * 1e3, 4),
            "encode_ms": round(te * 1e3, 4), "decode_ms": round(td * 1e3, 4),
            "encode_kv_GBs": round(N * esz / te / 1e9, 2), "decode_kv_GBs": round(N * esz / td / 1e9, 2),
            "encode_hbm_frac": round(alg / te / 1e9 / HBM_PEAK_GBS, 4),
            "decode_hbm_frac": round(alg / td / 1e9 / HBM_PEAK_GBS, 4), **fold}


def small_lines(steps, warmup):
    """small cache, fp32: zfp-4 and block-uniform 4-bit (32-token blocks), g = 16"""
    from fixed_rate_compression_amd import binding as cg
    lines = []
    L, KV, B, H, T = 1, 2, 1, 2, 4096
    x = _gen(L * KV * B * H, T, T, 0.9, 1, 2, False)
    G, _ = _gauge(L, KV, H, 16, 101)
    sh = cg.make_shape(L, KV, B, H, T, T, 128, cg.CG_DTYPE_F32)
    for codec, nm in ((cg.make_codec(cg.CG_BACKEND_ZFP, 4), "zfp4"),
                      (cg.make_codec(cg.CG_BACKEND_BLOCK_UNIFORM, 4, 32), "bu4")):
        lines.append(_codec_line(f"small_fp32_{nm}", sh, x, G, 16, codec, steps, warmup, 4,
                                 "1 layer x K/V x 2 heads x 4096 tokens fp32, g=16 (cache-resident)"))
    return lines


def llama8b_lines(steps, warmup):
    """Llama-3-8B-class cache at 3, 4 and 6 b/v with g = 16 (zfp-style,
    block-uniform and KIVI-style; with the error sums and the folded-recovery
    decodes), and zfp-style 4 b/v with the other groups"""
    import torch

    from fixed_rate_compression_amd import binding as cg
    lines = []
    L, KV, B, H, T = 32, 2, 1, 8, 32768
    x = _gen(L * KV * B * H, T, T, 0.95, 2, 4, True)
    G, _ = _gauge(L, KV, H, 16, 102)
    sh = cg.make_shape(L, KV, B, H, T, T, 128, cg.CG_DTYPE_BF16)
    for R in (3, 4, 6):
        lines.append(_codec_line(f"llama8b_zfp{R}", sh, x, G, 16, cg.make_codec(cg.CG_BACKEND_ZFP, R),
                                 steps, warmup, 2, "32 layers x K/V x 8 heads x 32768 tokens bf16, g=16"))
    for bits in (3, 4, 6):
        for codec, nm in ((cg.make_codec(cg.CG_BACKEND_BLOCK_UNIFORM, bits, 32), "bu"),
                          (cg.make_codec(cg.CG_BACKEND_KIVI, bits, 32, 128), "kivi")):
            lines.append(_codec_line(f"llama8b_{nm}{bits}", sh, x, G, 16, codec, steps, warmup, 2,
                                     "32 layers x K/V x 8 heads x 32768 tokens bf16, g=16"
                                     + (", 32-token blocks" if nm == "bu" else ", group 32, 128-token tail")))
    for g in (8, 32, 128):
        Gg, _ = _gauge(L, KV, H, g, 102 + g)
        lines.append(_codec_line(f"llama8b_zfp4_g{g}", sh, x, Gg, g, cg.make_codec(cg.CG_BACKEND_ZFP, 4),
                                 steps, warmup, 2, f"32 layers x K/V x 8 heads x 32768 tokens bf16, g={g}"
                                 + (" (dense, matrix cores)" if g == 128 else "")))
    del x
    torch.cuda.empty_cache()
    return lines


def llama8b_rate_lines(steps, warmup, rates=(3, 6)):
    """the other zfp rates of the Llama-3-8B-class cache (g = 16)"""
    import torch

    from fixed_rate_compression_amd import binding as cg
    L, KV, B, H, T = 32, 2, 1, 8, 32768
    x = _gen(L * KV * B * H, T, T, 0.95, 2, 4, True)
    G, _ = _gauge(L, KV, H, 16, 102)
    sh = cg.make_shape(L, KV, B, H, T, T, 128, cg.CG_DTYPE_BF16)
    lines = [_codec_line(f"llama8b_zfp{R}", sh, x, G, 16, cg.make_codec(cg.CG_BACKEND_ZFP, R), steps,
                         warmup, 2, "32 layers x K/V x 8 heads x 32768 tokens bf16, g=16", folded=False)
             for R in rates]
    del x
    torch.cuda.empty_cache()
    return lines


def fullhead_lines(steps, warmup, folded=True):
    """full-head gauge (g = 128, MFMA): KIVI-2/4 (group 32, 128-token tail), block-uniform 3-bit.
    Callers pass at least 3 warm-up launches: the first launches over these
    17 GB tensors run up to 20 % slower than the steady state (clocks and
    address-translation caches warming up)."""
    import torch

    from fixed_rate_compression_amd import binding as cg
    lines = []
    L, KV, B, H, T = 32, 2, 1, 8, 131072
    x = _gen(L * KV * B * H, T, T, 0.95, 3, 4, True)
    G, _ = _gauge(L, KV, H, 128, 103)
    sh = cg.make_shape(L, KV, B, H, T, T, 128, cg.CG_DTYPE_BF16)
    for codec, nm in ((cg.make_codec(cg.CG_BACKEND_KIVI, 2, 32, 128), "kivi2"),
                      (cg.make_codec(cg.CG_BACKEND_KIVI, 4, 32, 128), "kivi4"),
                      (cg.make_codec(cg.CG_BACKEND_BLOCK_UNIFORM, 3, 64), "bu3")):
        lines.append(_codec_line(f"fullhead_{nm}", sh, x, G, 128, codec, steps, warmup, 2,
                                 "32 layers x K/V x 8 heads x 131072 tokens bf16, dense g=128",
                                 folded=folded))
    del x
    torch.cuda.empty_cache()
    return lines


def rolling_line(modes=True, appends=256):
    """rolling history: 64 seq x 28 layers x 4 heads, 8192 -> 8192 + 256 tokens, g = 32, 4 b/v
    (modes=False: the workload's own mode only; appends < 256 times the first appends only)"""
    import torch

    from fixed_rate_compression_amd import binding as cg
    from fixed_rate_compression_amd.rolling import RollingHistory
    L, KV, B, H, T0, nsteps = 28, 2, 64, 4, 8192, appends
    cap = T0 + 256
    raw = _gen(L * KV * B * H, cap, cap, 0.95, 4, 4, True)
    G, _ = _gauge(L, KV, H, 32, 104)

    def run(every_token, keep):
        rh = RollingHistory(L, KV, B, H, cap, cg.make_gauge(32, G), 4, every_token=every_token, keep=keep)
        rh.prefill(raw, T0)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for k in range(nsteps):
            rh.append(raw[:, T0 + k])
        b.record()
        torch.cuda.synchronize()
        del rh
        torch.cuda.empty_cache()
        return a.elapsed_time(b) / nsteps

    ms = run(False, 0)                      # the workload: encode each completed 4-token block
    Nmean = L * KV * B * H * 128 * (T0 + nsteps / 2)
    line = {"workload": "rolling_g32_zfp4", "desc": "64 seq x 28 layers x 4 heads, history 8192+, "
            f"{nsteps} appends (encode each completed 4-token block, decode + inverse-gauge the whole history)",
            "ms_per_step": round(ms, 4), "history_values_mean": int(Nmean),
            "decode_kv_GBs": round(Nmean * 2 / (ms * 1e-3) / 1e9, 2),
            "decode_hbm_frac": round(Nmean * 2.5 / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if modes:
        line["ms_per_step_every_token"] = round(run(True, 0), 4)   # every token through the codec
        line["ms_per_step_every_token_folded"] = round(run(True, cg.CG_KEEP_KEYS | cg.CG_KEEP_VALUES), 4)
    del raw
    torch.cuda.empty_cache()
    return line


def b27_codec_line(steps, warmup, folded=True):
    """27B-class cache, zfp-3, g = 16"""
    import torch

    from fixed_rate_compression_amd import binding as cg
    L, KV, B, H, T = 46, 2, 1, 16, 65536
    x = _gen(L * KV * B * H, T, T, 0.95, 5, 4, True)
    G, _ = _gauge(L, KV, H, 16, 105)
    sh = cg.make_shape(L, KV, B, H, T, T, 128, cg.CG_DTYPE_BF16)
    line = _codec_line("27b_zfp3", sh, x, G, 16, cg.make_codec(cg.CG_BACKEND_ZFP, 3), steps, warmup, 2,
                       "46 layers x K/V x 16 heads x 65536 tokens bf16, g=16", folded=folded)
    del x
    torch.cuda.empty_cache()
    return line


def stats_line():
    """27B-class gauge-fit statistics over 64 x 4096-token windows of every head"""
    import torch

    from fixed_rate_compression_amd import binding as cg
    L, KV, B, H = 46, 2, 1, 16
    F = L * KV * B * H
    _, A = _gauge(L, KV, H, 16, 105)
    W, Tw = 64, 4096
    xw = _gen(F, W * Tw, W * Tw, 0.95, 205, 4, True, windows=W)
    shw = cg.make_shape(L, KV, B, H, W * Tw, W * Tw, 128, cg.CG_DTYPE_BF16)
    ws = torch.empty(cg.cg_stats_workspace_bytes(shw, 16, 16), dtype=torch.uint8, device="cuda")
    cg.cg_gauge_fit_stats(shw, xw, 16, A, 16, 0.04, 1.0, 0.02, ws, grad=True)
    t0 = time.perf_counter()
    st, dA = cg.cg_gauge_fit_stats(shw, xw, 16, A, 16, 0.04, 1.0, 0.02, ws, grad=True)
    wall = time.perf_counter() - t0
    t1 = time.perf_counter()
    cg.cg_gauge_fit_stats(shw, xw, 16, A, 16, 0.04, 1.0, 0.02, ws, grad=False)
    wall_nograd = time.perf_counter() - t1
    N = xw.numel()
    line = {"workload": "27b_stats_windows", "desc": "1472 heads x 64 windows x 4096 tokens bf16, "
            "g=16, T_b=16, tau=0.04; statistics + dL/dA (synchronous, includes the host exp and "
            "Frechet adjoint)",
            "values": N, "wall_s_with_grad": round(wall, 4), "wall_s_stats_only": round(wall_nograd, 4),
            "kv_GBs_with_grad": round(N * 2 / wall / 1e9, 2),
            "kv_GBs_stats_only": round(N * 2 / wall_nograd / 1e9, 2),
            "mean_L_freq": float(np.mean(st["L_freq"])), "mean_L": float(np.mean(st["L"]))}
    del xw
    torch.cuda.empty_cache()
    return line


WORKLOADS = ("small", "llama8b-rates", "fullhead", "rolling", "27b", "stats", "fit")


def workload_lines(names, steps, warmup, appends=256):
    lines = []
    for nm in names:
        if nm == "small":
            lines += small_lines(steps, warmup)
        elif nm == "llama8b-rates":
            lines += llama8b_lines(steps, warmup)
        elif nm == "fullhead":
            lines += fullhead_lines(max(3, steps // 4), 3)
        elif nm == "rolling":
            lines.append(rolling_line(appends=appends))
        elif nm == "27b":
            lines.append(b27_codec_line(steps, warmup))
        elif nm == "stats":
            lines.append(stats_line())
        elif nm == "fit":
            lines.append(fit_line())
    return lines


def fit_line(epochs=25):
    """Gauge training on synthetic windows and the zfp coordinate-control
    comparison: 2 layers x K/V x 8 heads, 16 training windows of 4096 tokens
    (AdamW, one step per window, 25 epochs, g = 16), 4 held-out windows; each
    condition's spectral concentration and zfp KV NRMSE at 3, 4, 6 b/v."""
    import torch

    from fixed_rate_compression_amd import fit
    L, KV, B, H, Tw, W, We = 2, 2, 1, 8, 4096, 16, 4
    x = _gen(L * KV * B * H, Tw * W, Tw * W, 0.95, 6, 4, True)
    held = _gen(L * KV * B * H, Tw * We, Tw * We, 0.95, 206, 4, True, scale_seed=6)  # same channel scales
    tr = fit.GaugeTrainer(x, L, KV, B, H, 16, window=Tw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tr.fit(epochs)
    t_fit = time.perf_counter() - t0
    conds = {"identity": None, "learned": tr.gauges(),
             "hadamard": fit.control_gauges("hadamard", L, KV, H, 16),
             "dct": fit.control_gauges("dct", L, KV, H, 16),
             "klt": fit.control_gauges("klt", L, KV, H, 16, moments=fit.second_moments(x, L, KV, B, H, 16))}
    for k in range(3):
        conds[f"random{k}"] = fit.control_gauges("random", L, KV, H, 16, seed=300 + k)
    res = {c: fit.evaluate(held, L, KV, B, H, 16, G) for c, G in conds.items()}
    out = {"workload": "gauge_fit_controls",
           "desc": f"{L} layers x K/V x {H} heads, g=16, AdamW {epochs} epochs x {W} windows of {Tw} tokens "
                   f"(one step per window), evaluated on {We} held-out windows (same channel scales, "
                   "new token noise)",
           "steps": tr.t, "fit_s": round(t_fit, 3), "ms_per_step": round(t_fit / tr.t * 1e3, 3),
           "objective_first_epoch": round(float(np.mean(tr.history[:W])), 6),
           "objective_last_epoch": round(float(np.mean(tr.history[-W:])), 6),
           "conditions": {c: {k: round(v, 6) for k, v in r.items()} for c, r in res.items()}}
    for R in (3, 4, 6):
        ident = res["identity"][f"zfp{R}_nrmse"]
        out[f"learned_vs_identity_zfp{R}_nrmse_reduction"] = round(1.0 - res["learned"][f"zfp{R}_nrmse"] / ident, 4)
    del x, held
    torch.cuda.empty_cache()
    return out


def config_summaries(steps, warmup):
    """Encode/decode figures of every other workload, measured in this run
    (medians of HIP-event times): the compact form of the --workload lines."""
    import torch

    keep = ("values", "bits_per_value", "encode_ms", "decode_ms", "encode_hbm_frac", "decode_hbm_frac",
            "kv_nrmse")

    def compact(line):
        return {k: line[k] for k in keep if k in line}

    out = {}
    log("configs: small fp32 cache")
    out["small_fp32_g16"] = {ln["workload"]: compact(ln) for ln in small_lines(steps, warmup)}
    log("configs: Llama-3-8B-class cache at 3 and 6 b/v")
    out["llama8b_g16_other_rates"] = {ln["workload"]: compact(ln)
                                      for ln in llama8b_rate_lines(steps, warmup)}
    log("configs: full-head gauge quantizers")
    out["fullhead_g128"] = {ln["workload"]: compact(ln)
                            for ln in fullhead_lines(max(3, steps // 2), 3, folded=False)}
    log("configs: rolling history")
    rl = rolling_line(modes=False)
    out["rolling_g32_zfp4"] = {k: rl[k] for k in ("ms_per_step", "history_values_mean", "decode_hbm_frac")}
    log("configs: 27B-class cache and its gauge-fit statistics")
    out["27b_g16"] = {"zfp3": compact(b27_codec_line(steps, warmup, folded=False))}
    st = stats_line()
    out["27b_g16"]["stats"] = {k: st[k] for k in ("values", "wall_s_with_grad", "wall_s_stats_only",
                                                   "kv_GBs_with_grad", "kv_GBs_stats_only")}
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads' figures (the `configs` key)")
    ap.add_argument("--workload", default="llama8b", choices=["llama8b", "all"] + list(WORKLOADS),
                    help="llama8b: the headline line only; all: the headline line, then one JSON "
                         "line per other workload; any other name: only that workload's lines")
    ap.add_argument("--appends", type=int, default=256,
                    help="rolling workload: appends timed (256 = the whole workload)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain device copy of the KV tensor (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the path shards "
              "by field with no exchange, so run one process per GPU on its own fields)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.workload in WORKLOADS:
        for line in workload_lines([args.workload], max(3, args.steps // 2), 1, args.appends):
            print(json.dumps(line), flush=True)
        return
    from fixed_rate_compression_amd import probe

    log("setup: generating the synthetic cache on the device")
    s = setup()
    if args.copy_probe:
        s["out"].copy_(s["x"])
        torch.cuda.synchronize()
    log(f"timing {args.steps} steps after {args.warmup} warmup")
    wall, enc, dec = time_steps(s, args.steps, args.warmup)
    N, R = s["N"], s["R"]
    kv_bytes = N * 2
    alg = N * 2 + N * R // 8            # read bf16 + write payload (and the reverse)
    t_enc, t_dec = float(np.median(enc)), float(np.median(dec))
    ms_step = (t_enc + t_dec) * 1e3
    value = kv_bytes / (t_enc + t_dec) / 1e9
    dom = "encode" if t_enc >= t_dec else "decode"
    t_dom = max(t_enc, t_dec)
    achieved = alg / t_dom / 1e9
    log("streaming-kernel memory ceiling")
    ceil = probe.ceilings(s["x"])
    ceil_dom = ceil["enc" if dom == "encode" else "dec"]["GBs"]
    alu = issue_slots(f"k_zfp_{dom}", t_dom)
    hbm_frac = round(achieved / HBM_PEAK_GBS, 4)
    # the resource the kernel is bound by: the one with the larger measured fraction
    bound = "alu" if alu["frac"] is not None and alu["frac"] > achieved / ceil_dom else "hbm"
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3-8B-class GQA KV cache round trip: 32 layers x K/V x 8 KV heads x "
                        "head_dim 128 x 32768 tokens, bf16 storage, gauge g=16, zfp-style 4 b/v",
            "values": N, "storage": "bf16", "gauge_group": s["g"], "zfp_rate": R,
            "compute": "fp32 gauge (matrix-core fmaf chains), int32 block coder",
            "global_batch": 1, "seq_len": s["T"], "parallelism": "none (1 GPU)",
            "timing": "median of HIP-event times per direction",
        },
        "encode": {"ms": round(t_enc * 1e3, 4), "kv_GBs": round(kv_bytes / t_enc / 1e9, 2),
                   "hbm_GBs": round(alg / t_enc / 1e9, 2),
                   "hbm_frac": round(alg / t_enc / 1e9 / HBM_PEAK_GBS, 4),
                   "frac_of_stream_ceiling": round(alg / t_enc / 1e9 / ceil["enc"]["GBs"], 4)},
        "decode": {"ms": round(t_dec * 1e3, 4), "kv_GBs": round(kv_bytes / t_dec / 1e9, 2),
                   "hbm_GBs": round(alg / t_dec / 1e9, 2),
                   "hbm_frac": round(alg / t_dec / 1e9 / HBM_PEAK_GBS, 4),
                   "frac_of_stream_ceiling": round(alg / t_dec / 1e9 / ceil["dec"]["GBs"], 4)},
        "bits_per_value": round(8.0 * (s["pbytes"] + s["hbytes"]) / N, 6),
        "wall_s": round(wall, 4),
        "roofline": {"bound": bound, "kernel": f"k_zfp_{dom}", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": hbm_frac,
                     "traffic": measured_traffic(f"k_zfp_{dom}"),
                     "alg_bytes_per_launch": alg,
                     "stream_ceiling_GBs": ceil_dom,
                     "frac_of_stream_ceiling": round(achieved / ceil_dom, 4),
                     "alu": alu},
        "stream_ceilings": ceil,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(s)
    del s
    torch.cuda.empty_cache()
    if not args.no_configs:
        res["configs"] = config_summaries(max(3, args.steps // 4), 1)
    print(json.dumps(res), flush=True)
    if args.workload == "all":
        for line in workload_lines(WORKLOADS, max(3, args.steps // 2), 1):
            print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
