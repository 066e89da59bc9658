"""python3 -m fixed_rate_compression_amd.probe issue: print the instruction-issue
rates and the matrix-core / VALU overlap times of issue.hip (one line each).
python3 -m fixed_rate_compression_amd.probe stream: print the streaming
kernels' HBM rates on a 4.29 GB tensor (stream.hip, every mode).
python3 -m fixed_rate_compression_amd.probe lds: print the times of the LDS
matrix-operand read patterns (lds.hip)."""
import sys

from fixed_rate_compression_amd import probe


def main() -> int:
    if len(sys.argv) < 2 or sys.argv[1] not in ("issue", "stream", "lds"):
        print(__doc__)
        return 2
    if sys.argv[1] == "lds":
        for name, ms in probe.lds_times().items():
            print(f"{name:36s} {ms:.3f} ms", flush=True)
        return 0
    if sys.argv[1] == "stream":
        import torch
        kv = torch.zeros(1 << 31, dtype=torch.bfloat16, device="cuda")
        for name, r in probe.ceilings(kv, names=tuple(probe.MODES)).items():
            print(f"{name:10s} {r['GBs']:8.1f} GB/s  {r['ms']:.4f} ms  ({r['bytes']} B)", flush=True)
        return 0
    for name, gps in probe.issue_rates().items():
        print(f"{name:34s} {gps:8.1f} G wave64 instr/s  ({gps / 614.4:.2f} per SIMD issue slot at 2.4 GHz)",
              flush=True)
    for name, ms in probe.overlap_times().items():
        print(f"{name:44s} {ms:.3f} ms", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
