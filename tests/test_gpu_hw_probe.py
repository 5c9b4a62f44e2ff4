"""The oracle's hardware-facing pieces against the hardware itself (GPU).

* The E4M3 codec: v_cvt_pk_fp8_f32 (the instruction the kernel casts P·S with) must give
  the oracle's round-to-nearest-even code for every |x| < 464 (beyond that the
  instruction returns NaN; P·S never exceeds 448).
* The matrix-core model used for the parity tolerance: v_mfma_f32_32x32x64_f8f6f4 on
  random sink-shaped E4M3 operands must match ``oracle.mfma_model`` bit for bit (a rare
  last-ulp difference is allowed: the model's handling of group-sum truncation is an
  approximation at the fp32 rounding level).
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import e4m3, mfma_model

from _gpu_util import device, say

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw_probe", "libhw_probe.so")


@pytest.fixture(scope="module")
def probe():
    lib = ctypes.CDLL(LIB)
    vp = ctypes.c_void_p
    lib.hw_probe_cvt_e4m3.argtypes = [vp, vp, ctypes.c_long, vp]
    lib.hw_probe_mfma_dots.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_int, vp]
    return lib


def _fp32_sweep():
    mant = np.arange(0, 1 << 23, 61, dtype=np.uint32)
    parts = [(((e + 127) << 23) | mant).view(np.float32) for e in range(-16, 9)]
    vals = e4m3.all_finite_values()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    parts += [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
              np.array([0.0, 448.0, 450.0, 463.9, 464.0, 1e-40, 2.0 ** -10], dtype=np.float32)]
    x = np.concatenate(parts)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 464]
    return x if x.size % 2 == 0 else x[:-1]


def test_hardware_cvt_matches_oracle_codec(probe):
    x = _fp32_sweep()
    say(f"case hw cvt sweep n={x.size}")
    dev = device()
    xin = torch.from_numpy(x).to(dev)
    out = torch.empty(x.size, dtype=torch.uint8, device=dev)
    assert probe.hw_probe_cvt_e4m3(xin.data_ptr(), out.data_ptr(), x.size, None) == 0
    torch.cuda.synchronize()
    hw = out.cpu().numpy()
    ref = e4m3.encode(x.astype(np.float64))
    bad = hw != ref
    assert not bad.any(), (x[bad][:8], hw[bad][:8], ref[bad][:8])


@pytest.mark.parametrize("kch", [1, 2, 4])
def test_hardware_mfma_matches_accumulation_model(probe, kch):
    T, K = 96, 64 * kch
    rng = np.random.default_rng(kch)
    scale = rng.choice([20.0, 60.0, 140.0], size=(T, 1, 1))
    a = rng.standard_normal((T, 32, K)) * scale
    b = rng.standard_normal((T, 32, K)) * scale
    a[:, :, 0] = 448.0
    b[:, :4, 0] = 448.0
    b[:, 4:, 0] = rng.standard_normal((T, 28)) * 300
    a8 = e4m3.encode(np.clip(a, -448, 448))
    b8 = e4m3.encode(np.clip(b, -448, 448))
    say(f"case hw mfma vs model kch={kch}")
    dev = device()
    ta = torch.from_numpy(a8).to(dev)
    tb = torch.from_numpy(b8).to(dev)
    raw = torch.empty((T, 32, 32), dtype=torch.float32, device=dev)
    assert probe.hw_probe_mfma_dots(ta.data_ptr(), tb.data_ptr(), raw.data_ptr(), T, kch, None) == 0
    torch.cuda.synchronize()
    hw = raw.cpu().numpy().astype(np.float64)
    model = np.stack([mfma_model.model_dots(a8[t], b8[t]) for t in range(T)])
    exact = np.einsum("tik,tjk->tij", e4m3.decode(a8), e4m3.decode(b8))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(hw), 1e-30))) - 23)
    same = hw == model
    say(f"  bit-exact {same.mean():.6f}; max|hw-model| {np.abs(hw - model).max():.3g}; "
        f"max|hw-exact| {np.abs(hw - exact).max():.3g}")
    assert same.mean() >= 0.999
    assert (np.abs(hw - model) <= ulp).all()
