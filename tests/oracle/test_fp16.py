"""Pins for oracle.fp16: the IEEE binary16 format and round-to-nearest-even."""
import numpy as np
import torch

from oracle import fp16


def test_exact_values_unchanged():
    vals = np.array([0.0, 1.0, -1.0, 0.5, 1.5, 3.0, 2.0 ** -14, 2.0 ** -24, 1.0 + 2.0 ** -10,
                     65504.0, -65504.0, 1024.0 + 1.0, 2.0 ** -24 * 1023])
    assert np.array_equal(fp16.round_to_f16(vals), vals)


def test_halfway_cases_round_to_even():
    u = 2.0 ** -10                        # fp16 spacing in [1, 2)
    cases = {1.0 + u / 2: 1.0,            # tie, 1.0 is even
             1.0 + 3 * u / 2: 1.0 + 2 * u,   # tie, 1+2u is even
             1.0 + u / 2 + 2.0 ** -40: 1.0 + u,  # just above the tie
             -(1.0 + u / 2): -1.0,
             2048.0 + 1.0: 2048.0,        # spacing 2 in [2048, 4096): tie to even
             2048.0 + 3.0: 2052.0,
             2.0 ** -24 / 2: 0.0,         # tie at the smallest subnormal -> even (zero)
             3 * 2.0 ** -25: 2.0 ** -23,  # subnormal tie -> even multiple of 2**-24
             65504.0 + 8.0: 65504.0,      # below the overflow tie (65520) stays finite
             65520.0: np.inf,             # tie between 65504 and 2**16 -> even -> overflow
             -65520.0: -np.inf}
    for x, want in cases.items():
        assert fp16.round_to_f16(np.float64(x)) == want, x


def test_matches_numpy_and_torch_conversions():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-20, 12, 200000))
    ours = fp16.f64_to_bits(x)
    with np.errstate(over="ignore"):
        assert np.array_equal(ours, x.astype(np.float16).view(np.uint16))
    x32 = x.astype(np.float32)
    ours32 = fp16.f64_to_bits(x32.astype(np.float64))
    theirs = torch.from_numpy(x32).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours32, theirs)


def test_bits_roundtrip():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    vals = fp16.bits_to_f64(bits)
    finite = np.isfinite(vals)
    assert np.array_equal(fp16.f64_to_bits(vals[finite]), bits[finite])
