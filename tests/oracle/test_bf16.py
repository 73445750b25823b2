"""Pins for oracle.bf16: the bfloat16 format and round-to-nearest-even."""
import numpy as np
import torch

from oracle import bf16


def test_exact_values_unchanged():
    vals = np.array([0.0, 1.0, -1.0, 0.5, 1.5, 3.0, 2.0 ** -126, 2.0 ** -133, 1.0 + 2.0 ** -7,
                     -(2.0 - 2.0 ** -7) * 2.0 ** 127])
    assert np.array_equal(bf16.round_to_bf16(vals), vals)


def test_halfway_cases_round_to_even():
    u = 2.0 ** -7                       # bf16 spacing in [1, 2)
    cases = {1.0 + u / 2: 1.0,           # tie, 1.0 is even
             1.0 + 3 * u / 2: 1.0 + 2 * u,  # tie, 1+2u is even
             1.0 + u / 2 + 2.0 ** -40: 1.0 + u,  # just above the tie
             -(1.0 + u / 2): -1.0,
             2.0 ** -133 / 2: 0.0,       # tie at the smallest subnormal -> even (zero)
             3 * 2.0 ** -134: 2.0 ** -132}
    for x, want in cases.items():
        assert bf16.round_to_bf16(np.float64(x)) == want, x


def test_matches_torch_fp32_to_bf16():
    rng = np.random.default_rng(0)
    x32 = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    ours = bf16.f64_to_bits(x32.astype(np.float64))
    theirs = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_bits_roundtrip():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16.bits_to_f64(bits)
    finite = np.isfinite(vals)
    back = bf16.f64_to_bits(vals[finite])
    # +0 / -0 both map back to themselves; every finite pattern is a fixed point
    assert np.array_equal(back, bits[finite])
