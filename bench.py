"""Benchmark: KV GB/s of the fused gauge + encode and decode + inverse-gauge
kernels at 4 bits/value, and their fraction of MI355X HBM bandwidth.

Workload (one GPU): a Llama-3-8B-class GQA cache, 32 layers x K/V x 8 KV
heads x head_dim 128 x 32768 tokens, bf16 storage, synthetic values
(lognormal channel scales, AR(1) rho = 0.95 along tokens, 4 outlier channels
at 20x per head), gauge g = 16 from A ~ N(0, 0.1^2), zfp-style fixed rate
4 bits/value.  One step = gauge + encode of the whole cache followed by
decode + inverse gauge of the whole cache; inputs are resident in HBM.

Prints one JSON line (see the repository's design doc for the fields).
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

CFG = dict(layers=32, kv=2, batch=1, heads=8, tokens=32768, head_dim=128, g=16, rate=4,
           rho=0.95, outliers=4, seed=2)


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


def cpu_baseline(s, n_fields=32):
    """The oracle (plain C + numpy, untuned) on a bounded sample of the same
    workload: n_fields fields (layers 0..1 of the cache), full round trip,
    one field per worker thread."""
    import concurrent.futures as cf

    import torch

    import oracle
    x = s["x"]
    D, T, R, g = s["D"], s["T"], s["R"], s["g"]
    L, KV, H = CFG["layers"], CFG["kv"], CFG["heads"]
    Gh = s["G"].cpu().numpy().reshape(L, KV, H, D // g, g, g)
    fields = list(range(min(n_fields, s["F"])))
    host = [x[f].view(torch.int16).cpu().numpy().view(np.uint16) for f in fields]
    threads = max(1, min(16, os.cpu_count() or 1, len(fields)))

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
    return dict(value=round(nvals * 2 / wall / 1e9, 4), unit="GB/s", cores=threads, kind="oracle",
                sample=f"{len(fields)} of {s['F']} fields ({nvals} values), gauge+encode+decode+"
                       f"inverse round trip, {wall:.2f} s wall on {threads} threads")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain device copy of the KV tensor (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the path shards "
              "by field with no exchange; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
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
    t_enc, t_dec = float(enc.mean()), float(dec.mean())
    ms_step = (t_enc + t_dec) * 1e3
    value = kv_bytes / (t_enc + t_dec) / 1e9
    dom = "encode" if t_enc >= t_dec else "decode"
    t_dom = max(t_enc, t_dec)
    achieved = alg / t_dom / 1e9
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
        "dtype": "f32+i32",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3-8B-class GQA KV cache round trip: 32 layers x K/V x 8 KV heads x "
                        "head_dim 128 x 32768 tokens, bf16 storage, gauge g=16, zfp-style 4 b/v",
            "values": N, "storage": "bf16", "gauge_group": s["g"], "zfp_rate": R,
            "global_batch": 1, "seq_len": s["T"], "parallelism": "none (1 GPU)",
        },
        "encode": {"ms": round(t_enc * 1e3, 4), "kv_GBs": round(kv_bytes / t_enc / 1e9, 2),
                   "hbm_GBs": round(alg / t_enc / 1e9, 2),
                   "hbm_frac": round(alg / t_enc / 1e9 / HBM_PEAK_GBS, 4)},
        "decode": {"ms": round(t_dec * 1e3, 4), "kv_GBs": round(kv_bytes / t_dec / 1e9, 2),
                   "hbm_GBs": round(alg / t_dec / 1e9, 2),
                   "hbm_frac": round(alg / t_dec / 1e9 / HBM_PEAK_GBS, 4)},
        "bits_per_value": round(8.0 * (s["pbytes"] + s["hbytes"]) / N, 6),
        "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": f"k_zfp_{dom}", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "alg_bytes_per_launch": alg},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(s)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
