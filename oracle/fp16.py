"""IEEE binary16 (fp16) storage format for the oracle (test infrastructure only).

A widening of the storage formats: the pages fix bf16 (Chelsea review, section 五, 实验设置
默认配置), and the method (Algorithm 1) does not depend on the format, so the cache may be
stored in fp16 as well.  binary16: 1 sign bit, 5 exponent bits (bias 15), 10 stored
fraction bits (11 significant bits); normal numbers from 2**-14 to 65504, subnormals with a
fixed spacing of 2**-24.  Rounding from a wider value is round-to-nearest, ties-to-even;
magnitudes that round above 65504 become infinities.

Pins (tests/oracle/test_fp16.py): exact values stay unchanged; hand-built halfway cases
round to the even neighbour, in the normal and the subnormal range and at the overflow
threshold; random fp64 inputs agree with numpy's float64 -> float16 conversion.
"""

import numpy as np

F16_MAX = 65504.0


def round_to_f16(x):
    """Nearest fp16 value of fp64 ``x`` (ties to even), returned as fp64.

    For |x| in [2**(e-1), 2**e) the fp16 grid spacing is 2**(e-11); below the smallest
    normal (2**-14) the spacing is fixed at 2**-24, i.e. e is clamped at -13.  Dividing by a
    power of two is exact in fp64 and numpy's rint rounds halves to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -13)
    scale = np.ldexp(1.0, e - 11)
    out = np.rint(x / scale) * scale
    out = np.where(np.abs(out) > F16_MAX, np.copysign(np.inf, x), out)
    return out


def bits_to_f64(bits):
    """uint16 fp16 bit patterns -> exact fp64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_bits(x):
    """fp64 -> fp16 bit patterns (uint16), rounding to nearest even."""
    return round_to_f16(x).astype(np.float16).view(np.uint16)
