"""Pins of the closed forms (CPU only): each against the pages' printed numbers,
Monte Carlo, brute force or exhaustive fp32 enumeration."""
import json
import math
import os

import numpy as np
import pytest

from oracle import e4m3, theory

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def test_delta_4_quadrature_vs_monte_carlo_and_pages():
    d4 = theory.delta_k(4)
    rng = np.random.default_rng(0)
    mx = rng.standard_normal((2_000_000, 4)).max(axis=1)
    se = mx.std() / math.sqrt(mx.size)
    assert abs(d4 - mx.mean()) < 4 * se
    assert abs(theory.var_max_k(4) - mx.var()) < 2e-3
    assert abs(d4 - GOLD["delta_4"]["value"]) < 0.05            # printed "≈ 1.0"
    assert abs(theory.delta_k(1)) < 1e-10                         # max of one is the mean
    assert abs(theory.delta_k(2) - 1 / math.sqrt(math.pi)) < 1e-9  # textbook E[max of 2]


def test_ln_threshold_is_ten_ln2():
    assert abs(theory.LN_ZERO - GOLD["ln_zero_threshold"]["value"]) < 0.005
    assert math.isclose(math.exp(-theory.LN_ZERO), GOLD["e4m3_zero_threshold"]["value"])


def test_collapse_fraction_formula_and_threshold():
    # F at Δ_c is exactly 1/2; F rises with Δ and falls with S
    for S in (1, 16, 256, 448):
        dc = theory.collapse_threshold(S)
        assert abs(theory.collapse_fraction(dc, S) - 0.5) < 1e-12
        assert math.isclose(dc, 6.931471805599453 + math.log(S) - theory.delta_k(4))
    d = np.linspace(0, 14, 57)
    assert (np.diff(theory.collapse_fraction(d, 256)) > 0).all()
    assert theory.collapse_fraction(8, 1) > theory.collapse_fraction(8, 16) > theory.collapse_fraction(8, 256)
    # printed onset: for S = 1 the threshold sits at Δ ≈ 6–7 (within the printed rounding)
    lo, hi = GOLD["collapse_onset_delta"]["value"]
    assert lo - 0.25 <= theory.collapse_threshold(1) <= hi
    # with the printed constants 6.93 and δ_4 = 1.0 the formula moves by < 0.04 in probit
    for D in (6, 8, 10):
        z_exact = D + theory.delta_k(4) - theory.LN_ZERO - math.log(256)
        z_print = D + 1.0 - 6.93 - math.log(256)
        assert abs(z_exact - z_print) < 0.04


def test_collapse_fraction_vs_monte_carlo_of_its_own_model():
    """F(Δ,S) is the probability that a N(0,1) logit x satisfies exp(x - m)·S <= 2^-10
    with m = Δ + δ_4 (the sink block's expected max). Sample that event directly."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal(4_000_000)
    for D, S in [(7, 1), (8, 16), (12, 256), (12, 448)]:
        m = D + theory.delta_k(4)
        emp = np.mean(np.exp(x - m) * S <= 2.0 ** -10)
        assert abs(emp - theory.collapse_fraction(D, S)) < 2e-3


def test_reverse_bound_matches_pages():
    p = theory.reverse_order_underflow_bound(GOLD["reverse_bound_n"]["value"], GOLD["reverse_bound_scale"]["value"])
    assert p < GOLD["reverse_bound_prob"]["value"]
    # the bound needs S as well as the order: with S = 1 it is far above 1e-12
    assert theory.reverse_order_underflow_bound(1e6, 1) > 1e-6


def test_dp_sawtooth_bruteforce():
    env = GOLD["dp_lower_envelope"]["value"]
    for k in range(0, 9):
        assert theory.dp_bruteforce(2.0 ** k) == env
        assert theory.dp_closed_form(2.0 ** k) == env
    r448 = theory.dp_bruteforce(448.0)
    assert r448 == theory.dp_closed_form(448.0) == 1.0 / 14.0
    assert round(r448 / env - 1.0, 2) == GOLD["dp_448_excess"]["value"]
    # sawtooth: just above a power of two the step doubles, then decays to 2^-4
    assert theory.dp_bruteforce(257.0) > 0.12
    grid = [2.0 ** 7 * (1 + i / 16) for i in range(1, 17)]
    vals = [theory.dp_bruteforce(s) for s in grid]
    assert all(a >= b for a, b in zip(vals, vals[1:])) and vals[-1] == env
    assert min(theory.dp_bruteforce(s) for s in np.linspace(2, 448, 223)) >= env


def test_largest_scale_and_normal_floor():
    assert theory.largest_pow2_scale() == 256
    assert e4m3.E4M3_MIN_NORMAL / 256 == GOLD["normal_floor_s256"]["value"] == 2.0 ** -14


@pytest.mark.parametrize("S", [1.0, 2.0, 16.0, 256.0])
def test_pow2_scale_roundtrip_exact_over_a_binade(S):
    """Every fp32 in [1, 2) and in [2^-20, 2^-19): x·S/S == x exactly for S = 2^k."""
    mant = np.arange(1 << 23, dtype=np.uint32)
    for e in (0, -20):
        x = (((e + 127) << 23) | mant).view(np.float32)
        assert theory.fp32_roundtrip_failures(S, x) == 0.0


def test_448_scale_roundtrip_drifts():
    mant = np.arange(1 << 23, dtype=np.uint32)
    x = ((127 << 23) | mant).view(np.float32)
    assert theory.fp32_roundtrip_failures(448.0, x) > 0.01
    # the epilogue multiply by fl(1/448) instead of a divide drifts as well
    inv = np.float32(1.0) / np.float32(448.0)
    assert np.mean((x * np.float32(448.0)) * inv != x) > 0.01
