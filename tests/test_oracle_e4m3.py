"""Pins of the oracle's E4M3 / bf16 codecs (CPU only).

The codec is checked against (a) the format constants the P-Cast pages print and
(b) torch's float8_e4m3fn / bfloat16 casts, an independent library implementation.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def test_decode_matches_printed_constants():
    # largest finite 448, smallest normal 2^-6, zero threshold 2^-10 (half the min subnormal)
    assert e4m3.decode(np.uint8(0x7E)) == GOLD["e4m3_max"]["value"]
    assert e4m3.decode(np.uint8(0x08)) == GOLD["e4m3_min_normal"]["value"]
    assert e4m3.decode(np.uint8(0x01)) / 2 == GOLD["e4m3_zero_threshold"]["value"]
    # 3 mantissa bits: 8 codes per binade, evenly spaced
    normal = e4m3.decode(np.arange(0x38, 0x40, dtype=np.uint8))
    assert GOLD["e4m3_mantissa_bits"]["value"] == 3
    assert np.allclose(np.diff(normal), 1.0 / 8) and normal[0] == 1.0
    assert np.isnan(e4m3.decode(np.uint8(0x7F))) and np.isnan(e4m3.decode(np.uint8(0xFF)))
    # the largest non-overflowing power of two scale is 256 and 512 would overflow
    assert 256 <= e4m3.E4M3_MAX < GOLD["overflow_scale"]["value"]


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3.decode(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), codes[~same]


def _fp32_binade_sweep(lo_exp, hi_exp, stride):
    """Every ``stride``-th fp32 mantissa of every binade [2^lo_exp, 2^hi_exp)."""
    mant = np.arange(0, 1 << 23, stride, dtype=np.uint32)
    out = []
    for e in range(lo_exp, hi_exp):
        bits = ((e + 127) << 23) | mant
        out.append(bits.view(np.float32))
    return np.concatenate(out)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_encode_matches_torch_dense_sweep(sign):
    x = sign * _fp32_binade_sweep(-14, 9, 13)          # [2^-14, 2^9) minus the overflow range
    x = x[np.abs(x) < 464]                             # torch's cast is NaN from 464 on
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3.encode(x.astype(np.float64))
    bad = got != ref
    assert not bad.any(), (x[bad][:5], got[bad][:5], ref[bad][:5])


def test_encode_ties_and_neighbours_of_every_midpoint():
    vals = e4m3.all_finite_values()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)     # exact in fp32
    x = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (e4m3.encode(x.astype(np.float64)) == ref).all()
    # ties go to the even code
    tie_codes = e4m3.encode(mids.astype(np.float64))
    assert (tie_codes % 2 == 0).all()


def test_zero_threshold_is_two_to_minus_ten():
    t = GOLD["e4m3_zero_threshold"]["value"]
    assert e4m3.encode(t) == 0                                  # the tie rounds to even 0
    assert e4m3.encode(np.nextafter(t, 1.0)) == 0x01            # anything above -> 2^-9
    x = np.geomspace(1e-6, 1e-2, 200001)
    assert ((e4m3.encode(x) == 0) == (x <= t)).all()
    assert e4m3.E4M3_ZERO_THRESHOLD == t


def test_saturation_and_roundtrip():
    assert e4m3.encode(448.0 * 1.03) == 0x7E
    assert e4m3.encode(-1e6) == 0xFE
    assert np.isnan(e4m3.round_e4m3(1e6, saturate=False))
    codes = np.concatenate([np.arange(0x7F), np.arange(0x80, 0xFF)]).astype(np.uint8)
    assert (e4m3.encode(e4m3.decode(codes)) == codes).all()


def test_bf16_matches_torch():
    x = np.concatenate([_fp32_binade_sweep(-30, 2, 997), -_fp32_binade_sweep(-3, 0, 1001)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert (e4m3.round_bf16(x.astype(np.float64)) == ref).all()
