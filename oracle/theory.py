"""Closed forms from the P-Cast analysis, evaluated in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

P-Cast technical summary ("P-Cast Precision in FP8 Attention", gist.science):
  * §2 Theoretical framework: under forward KV order the fraction of non-sink P that
    underflow is F(Δ, S) = Φ(Δ + δ_k − 6.93 − ln S), where Δ is the sink strength (logit
    gap), δ_k the expected maximum of k standard Gaussians in the sink block (≈ 1.0 for
    k = 4), 6.93 ≈ 10 ln 2 the log of the E4M3 zero threshold 2^-10, Φ the normal CDF.
  * §3 Contributions, item 1: the collapse threshold Δ_c = 6.93 + ln S − δ_k.
  * §2 Optimization 1: with reverse order the running max before the sink block is set
    by non-sink tokens only; for N <= 10^6 and S = 256 the chance that any non-sink P
    underflows is below 10^-12.
  * §2 Optimization 2: (1) S = 2^k makes the scale and the epilogue division exact in
    fp32, S = 448 does not; (2) the normalised maximum quantization step d_p(S) is a
    sawtooth whose lower envelope 2^-4 is reached at S = 2^k, with S = 448 14% above it;
    (3) among non-overflowing powers of two (S <= 448) S = 256 is the largest and
    reaches P = 2^-6/256 = 2^-14 in the normal range.

Here 6.93 is taken as exactly 10 ln 2 (the pages give the rounded value).
"""
from __future__ import annotations

import math

import numpy as np
from scipy import integrate, stats

from . import e4m3

LN_ZERO = 10.0 * math.log(2.0)          # -ln(2^-10): the E4M3 round-to-zero threshold


def phi_cdf(x):
    return stats.norm.cdf(x)


def delta_k(k: int) -> float:
    """E[max of k iid N(0,1)] = ∫ x · k φ(x) Φ(x)^(k-1) dx (numerical quadrature)."""
    f = lambda x: x * k * stats.norm.pdf(x) * stats.norm.cdf(x) ** (k - 1)
    val, _ = integrate.quad(f, -np.inf, np.inf, epsabs=1e-13, epsrel=1e-12)
    return val


def var_max_k(k: int) -> float:
    """Var[max of k iid N(0,1)]."""
    f = lambda x: x * x * k * stats.norm.pdf(x) * stats.norm.cdf(x) ** (k - 1)
    m2, _ = integrate.quad(f, -np.inf, np.inf, epsabs=1e-13, epsrel=1e-12)
    return m2 - delta_k(k) ** 2


def collapse_fraction(delta, S, k: int = 4):
    """F(Δ, S) = Φ(Δ + δ_k − 10 ln 2 − ln S): forward-order non-sink underflow fraction."""
    return phi_cdf(np.asarray(delta, dtype=np.float64) + delta_k(k) - LN_ZERO - np.log(S))


def collapse_threshold(S, k: int = 4):
    """Δ_c = 10 ln 2 + ln S − δ_k: the sink strength at which F = 1/2."""
    return LN_ZERO + np.log(S) - delta_k(k)


def collapse_fraction_rowwise(row_max, mu, sigma, S):
    """Per-row version of the same Gaussian tail: a non-sink logit x ~ N(mu_i, sigma_i)
    underflows when exp(x − m_i)·S <= 2^-10, i.e. x <= m_i − 10 ln 2 − ln S. Averages
    Φ((m_i − 10 ln 2 − ln S − mu_i)/sigma_i) over rows (m_i: the row's realised max)."""
    z = (np.asarray(row_max) - LN_ZERO - math.log(S) - np.asarray(mu)) / np.asarray(sigma)
    return float(np.mean(phi_cdf(z)))


def reverse_order_underflow_bound(n: float, S: float) -> float:
    """Reverse order: before the sink block the running max is that of non-sink logits,
    about sqrt(2 ln N) for N standard Gaussians. A non-sink logit underflows only if it
    lies 10 ln 2 + ln S below that max, probability Φ(sqrt(2 ln N) − 10 ln 2 − ln S)."""
    return float(phi_cdf(math.sqrt(2.0 * math.log(n)) - LN_ZERO - math.log(S)))


def e4m3_spacing_at(y):
    """Distance from the E4M3 value at/below y to the next one up (by enumeration)."""
    vals = e4m3.all_finite_values()
    y = np.asarray(y, dtype=np.float64)
    i = np.clip(np.searchsorted(vals, y, side="right") - 1, 0, len(vals) - 2)
    return vals[i + 1] - vals[i]


def dp_bruteforce(S: float, n: int = 200001) -> float:
    """d_p(S): the largest E4M3 quantization step met by P·S for P in [1/2, 1), divided
    by S (the step in the P domain, for the top octave of probabilities). Evaluated on a
    dense grid against the enumerated E4M3 values."""
    p = np.linspace(0.5, 1.0, n, endpoint=False)
    return float(np.max(e4m3_spacing_at(p * S)) / S)


def dp_closed_form(S: float) -> float:
    """For S in (2^(k-1), 2^k], P·S reaches the binade [2^(k-1), 2^k) whose E4M3 step is
    2^(k-4): d_p(S) = 2^(ceil(log2 S) - 4) / S. Equal to 2^-4 exactly at S = 2^k."""
    return 2.0 ** (math.ceil(math.log2(S)) - 4) / S


def largest_pow2_scale(max_finite: float = e4m3.E4M3_MAX) -> float:
    """Largest S = 2^k with S <= the E4M3 maximum (no overflow of P·S for P <= 1)."""
    return 2.0 ** math.floor(math.log2(max_finite))


def fp32_roundtrip_failures(S: float, x: np.ndarray) -> float:
    """Fraction of fp32 values x for which fl32(fl32(x·S)/S) != x (IEEE fp32, RNE)."""
    x = np.asarray(x, dtype=np.float32)
    s32 = np.float32(S)
    y = (x * s32) / s32
    return float(np.mean(y != x))
