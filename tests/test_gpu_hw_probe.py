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
    lib.hw_probe_throughput.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp]
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


def test_throughput_roofline_denominators(probe):
    """The measured ceilings the kernel's roofline fraction is read against: the FP8
    matrix-core rate of a pure v_mfma_f32_32x32x64_f8f6f4 stream, the v_exp_f32 rate, how
    far the two overlap (same wave, and split across the two waves of a SIMD), and the
    shader clock they ran at (printed; loose sanity bounds only)."""
    dev = device()
    blocks, iters = 1024, 2000
    seed = torch.from_numpy(np.random.default_rng(0).integers(0, 2**31 - 1, 256).astype(np.int32)).to(dev)
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    clock = torch.empty(blocks, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for kind, name in ((0, "mfma"), (1, "exp"), (2, "mfma+exp same wave"), (3, "mfma | exp split waves")):
        for rep in range(2):      # first launch warms up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            assert probe.hw_probe_throughput(kind, blocks, iters, seed.data_ptr(), sink.data_ptr(),
                                             clock.data_ptr(), ctypes.c_void_p(stream.cuda_stream)) == 0
            e1.record(stream)
            torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        ghz = float(clock.median()) * 0.1
        waves = blocks * 8 * (0.5 if kind == 3 else 1.0)
        flop = waves * iters * 8 * 2 * 32 * 32 * 64 if kind != 1 else 0.0
        exps = blocks * 8 * (0.5 if kind == 3 else 1.0) * iters * 32 * 64 if kind != 0 else 0.0
        tflops, texp = flop / ms / 1e9, exps / ms / 1e9
        res[name] = (ms, tflops, texp, ghz)
        per_clk = f"{flop / (ms * 1e-3) / (ghz * 1e9) / 1024:.0f} FLOP/clk/SIMD" if flop else \
            f"{exps / (ms * 1e-3) / (ghz * 1e9) / 256:.1f} exp/clk/CU"
        say(f"  {name:24s} {ms:8.3f} ms  {tflops:8.1f} TFLOP/s  {texp:6.2f} Texp/s  clock {ghz:.2f} GHz  {per_clk}")
    assert 1.0 < res["mfma"][3] < 2.7
    assert res["mfma"][1] > 2000.0              # FP8 MFMA stream well above 40% of 5.0 PF
    # the exp work hides under the MFMA work when both come from the same wave
    assert res["mfma+exp same wave"][0] < 1.5 * res["mfma"][0]
