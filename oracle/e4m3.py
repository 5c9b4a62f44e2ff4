"""OCP E4M3 ("e4m3fn") and bfloat16 codecs in fp64.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain CPU oracle for the FP8
P-cast attention forward. Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import it; the HIP library never does, and shares no code with it.

Format facts taken from the P-Cast technical summary ("P-Cast Precision in FP8
Attention: Sink-Induced Collapse and the Optimality of S=2^8", gist.science):
  * §1 Problem statement: E4M3 has a 3-bit mantissa.
  * §2 Theoretical framework: values at or below 2^-10 round to zero
    (the "6.93 = 10 ln 2" term of F(Δ,S)).
  * §2 Optimization 2, condition 3: the smallest normal is 2^-6 and the largest
    finite value is 448 (a power-of-two scale S must satisfy S <= 448).
Those three facts fix the OCP E4M3FN variant: exponent bias 7, no infinities,
the single NaN pattern S.1111.111, largest finite 0x7E = 448.

Rounding is round-to-nearest, ties-to-even (the 2^-10 zero threshold is half the
smallest subnormal 2^-9, i.e. a round-to-nearest cast; an exact tie goes to the even
code 0). Values above 448 saturate to 448 when ``saturate`` is true.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_MIN_SUBNORMAL = 2.0 ** -9
E4M3_ZERO_THRESHOLD = 2.0 ** -10      # x <= this rounds to 0 (tie -> even code 0)
E4M3_NAN_CODES = (0x7F, 0xFF)


def decode(codes) -> np.ndarray:
    """E4M3FN byte codes -> fp64 values.

    Bit layout s.eeee.mmm. Exponent field 0 is subnormal: m/8 * 2^-6. Otherwise
    (1 + m/8) * 2^(e-7). The patterns 0x7F and 0xFF are NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0,
                   (m / 8.0) * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def round_e4m3(x, saturate: bool = True) -> np.ndarray:
    """Round fp64 values to the nearest E4M3FN value (ties to even), as fp64.

    In the binade [2^e, 2^(e+1)) with e >= -6 the spacing is 2^(e-3); below 2^-6
    the spacing is the subnormal step 2^-9. Dividing by the spacing (a power of two,
    so exact) and rounding to the nearest integer with ties to even selects the
    neighbour with the even mantissa. Magnitudes above 448 saturate to 448
    (``saturate``) or become NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    spacing = np.exp2((np.maximum(ex, -5) - 4).astype(np.float64))
    r = np.rint(a / spacing) * spacing
    over = r > E4M3_MAX
    r = np.where(over, E4M3_MAX if saturate else np.nan, r)
    r = np.where(np.isnan(a), np.nan, r)
    return np.copysign(r, x)


def encode(x, saturate: bool = True) -> np.ndarray:
    """fp64 values -> E4M3FN byte codes (RNE; saturating to 0x7E/0xFE by default)."""
    r = round_e4m3(x, saturate=saturate)
    a = np.abs(r)
    sign = np.where(np.signbit(r), 0x80, 0).astype(np.int64)
    f, ex = np.frexp(a)
    # normal: a = (1 + m/8) * 2^(E-7) with f = (1 + m/8)/2 and ex - 1 = E - 7
    normal_code = ((ex + 6) << 3) + np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)
    sub_code = np.rint(a / E4M3_MIN_SUBNORMAL).astype(np.int64)   # 0..8 (8 is 2^-6)
    code = np.where(a < E4M3_MIN_NORMAL, np.where(np.isfinite(a), sub_code, 0), normal_code)
    code = np.where(np.isnan(a), 0x7F, code)
    return (code | sign).astype(np.uint8)


def all_finite_values() -> np.ndarray:
    """The 127 non-negative finite E4M3FN values, ascending (codes 0x00..0x7E)."""
    return decode(np.arange(0x7F, dtype=np.uint8))


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value (ties to even), as fp64.

    bfloat16 keeps 8 significant bits and fp32's exponent range: spacing 2^(e-7) in
    the binade [2^e, 2^(e+1)), and the fixed subnormal spacing 2^-133 below 2^-126.
    Used for the bf16 FlashAttention comparison, where P is rounded to bf16.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)
    spacing = np.exp2((np.maximum(ex, -125) - 8).astype(np.float64))
    r = np.rint(a / spacing) * spacing
    return np.copysign(r, x)
