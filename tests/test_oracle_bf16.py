"""Pin of the oracle's storage-format conversion: fp32 -> bf16 round to
nearest, ties to even (checked on hand-picked tie cases and against torch's
CPU conversion, an independent implementation), bf16 -> fp32 exact."""
import numpy as np
import torch

import oracle


def test_ties_and_carries_by_hand():
    # bit patterns: keep = top 16 bits, rest = low 16 bits
    cases = {
        0x3F808000: 0x3F80,  # tie, keep even -> stays
        0x3F818000: 0x3F82,  # tie, keep odd -> rounds up
        0x3F808001: 0x3F81,  # above half -> up
        0x3F807FFF: 0x3F80,  # below half -> down
        0x3FFF8000: 0x4000,  # tie on odd with carry into the exponent
        0x00008000: 0x0000,  # subnormal tie to even
        0x80018000: 0x8002,  # negative tie on odd
    }
    for bits, want in cases.items():
        f = np.array([bits], np.uint32).view(np.float32)
        assert int(oracle.f32_to_bf16(f)[0]) == want, hex(bits)


def test_matches_torch_cpu_and_exact_widening():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(8 * rng.standard_normal(200000))).astype(np.float32)
    x[:1000] = np.frombuffer(rng.integers(0, 2**32, 1000, dtype=np.uint64).astype(np.uint32).tobytes(), np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.0e38)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(x)
    assert np.array_equal(got, ref)
    back = oracle.bf16_to_f32(got)
    assert np.array_equal(back.view(np.uint32), got.astype(np.uint32) << 16)
