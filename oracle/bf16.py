"""bfloat16 storage format for the oracle (test infrastructure only).

The Chelsea review lists BFloat16 as the default numeric format (section 五, 实验设置
默认配置).  bfloat16 is the top 16 bits of an IEEE binary32: 1 sign bit, 8 exponent bits,
7 stored fraction bits (8 significant bits).  Rounding from a wider value is
round-to-nearest, ties-to-even.

Pins (tests/oracle/test_bf16.py): exact values stay unchanged; hand-built halfway cases
round to the even neighbour; fp32 inputs agree with torch's fp32->bf16 conversion.
"""

import numpy as np

_BF16_MAX = float(np.ldexp(2.0 - 2.0 ** -7, 127))


def round_to_bf16(x):
    """Nearest bfloat16 value of fp64 ``x`` (ties to even), returned as fp64.

    For |x| in [2**(e-1), 2**e) the bf16 grid spacing is 2**(e-8); below the smallest
    normal (2**-126) the spacing is fixed at 2**-133.  Dividing by a power of two is
    exact in fp64, and numpy's rint rounds halves to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    scale = np.ldexp(1.0, e - 8)
    out = np.rint(x / scale) * scale
    out = np.where(np.abs(out) > _BF16_MAX, np.copysign(np.inf, x), out)
    return out


def bits_to_f64(bits):
    """uint16 bf16 bit patterns -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bits(x):
    """fp64 -> bf16 bit patterns (uint16), rounding to nearest even."""
    r = round_to_bf16(x).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_to_storage(x, storage):
    """Round fp64 ``x`` to the cache storage format: 'bf16', 'f16', 'f32' (RNE) or 'f64'
    (none)."""
    if storage == "bf16":
        return round_to_bf16(x)
    if storage == "f16":
        from .fp16 import round_to_f16
        return round_to_f16(x)
    if storage == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if storage == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown storage format {storage!r}")
