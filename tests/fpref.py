"""A second, independent model of element rounding, used only to pin the oracle.

It follows the two-step floating-point quantiser of the LLM-FP4 summary page
("Floating-Point Quantization Mechanics"): clip to Q_max, find the binade of the
clipped value, take the step v = 2^(floor(log2 x) - m) of that binade (the
subnormal floor 2^(1 - bias - m) below the smallest normal), and round x / v to
an integer with ties to even.  It shares nothing with the oracle's
sorted-table binary search: there is no table and no search, only the step
formula, evaluated with numpy in float64 (exact for every value used here).
"""
import numpy as np

# (exponent bits, mantissa bits, bias, Q_max).  Q_max of OCP E4M3 is 448: the
# all-ones code is NaN, so the P4 formula's 480 is one step beyond the range.
E2M1 = (2, 1, 1, 6.0)
E4M3 = (4, 3, 7, 448.0)
# the unsigned scale grids of the qwantize "Exotic Scales" section: every code
# finite, so Q_max is the P4 formula's value
UE4M4 = (4, 4, 7, 496.0)
UE5M3 = (5, 3, 15, 122880.0)


def p4_value(ebits, mbits, bias, p, d):
    """Value of exponent field p and mantissa field d (P4's value formula,
    with the usual subnormal reading for p = 0)."""
    if p == 0:
        return np.ldexp(d / 2.0 ** mbits, 1 - bias)
    return np.ldexp(1.0 + d / 2.0 ** mbits, p - bias)


def p4_qmax(ebits, mbits, bias):
    """Q_max = (2 - 2^-m) * 2^(2^e - b - 1) of the LLM-FP4 summary page."""
    return (2.0 - 2.0 ** -mbits) * 2.0 ** (2 ** ebits - bias - 1)


def p4_round(x, fmt):
    """Round x >= 0 (array) onto the grid of fmt, saturating at Q_max."""
    ebits, mbits, bias, qmax = fmt
    x = np.minimum(np.asarray(x, np.float64), qmax)
    _, ex = np.frexp(x)                 # x = f * 2^ex, f in [0.5, 1)
    E = np.maximum(ex - 1, 1 - bias)    # binade exponent, floored at the subnormal range
    v = np.ldexp(1.0, E - mbits)        # step of that binade
    return np.rint(x / v) * v           # np.rint: ties to even


def int_round(x, qmax):
    """Symmetric integer grid 0..qmax: round half to even, then clip."""
    return np.minimum(np.rint(np.asarray(x, np.float64)), qmax)


def grid(ebits, mbits, bias, reserve_top_code):
    """All non-negative values of the format by direct enumeration of (p, d)."""
    vals = []
    for p in range(2 ** ebits):
        for d in range(2 ** mbits):
            if reserve_top_code and p == 2 ** ebits - 1 and d == 2 ** mbits - 1:
                continue
            vals.append(p4_value(ebits, mbits, bias, p, d))
    return np.array(vals)


def all_positive_bf16():
    """Every finite non-negative bfloat16 value, as float32."""
    b = np.arange(0, 0x7F80, dtype=np.uint32) << 16
    return b.view(np.float32)


def binade_f32(e0, e1):
    """Every float32 in [2^e0, 2^e1) as float32 (normal range only)."""
    out = []
    for e in range(e0, e1):
        base = np.uint32((e + 127) << 23)
        out.append((base + np.arange(1 << 23, dtype=np.uint32)).view(np.float32))
    return np.concatenate(out)
