"""Sequence-length and scale sweeps on the GPU: the output error of the HIP path against
exact fp64 attention on the fp32 source tensors, on sampled rows, for the pages' claims
that survive E4M3 quantisation of Q, K and V (the pages measure with Q, K, V in fp32).

* The gain of reverse order with S = 256 over forward order with S = 1 grows with the
  sequence length (technical summary, section 4 "Results", last point).
* Within each octave of S the power of two has the smaller error (the sawtooth of the
  normalised quantisation step d_p, section 2 "Optimization 2", condition 2).
* The quantized row-sum denominator (fp8_attn_fwd_ex) is no worse where nothing
  collapses and much worse where P collapses: the collapsed mass leaves the denominator
  too, so the sinks take the weight.
* The sink-last schedule changes the error of clean inputs by less than 1%.
* S = 256 against S = 384 and 448 in forward order, measured on the error the P cast adds
  (the GPU output against attention of the same E4M3 operands without the cast, the
  quantity the pages' comparison is about: section 4, "Scale comparison"). The size of the
  gain depends on where the large P~ fall within an octave; on this recipe the oracle gives
  3-6%, the pages print 10-15% for their own, unstated, P distribution.
Every measured table is printed (``-s`` shows it).
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import e4m3
from precision_attention_amd import binding
from precision_attention_amd import inputs as I

from _gpu_util import say, to_device

pytestmark = pytest.mark.gpu

D = 128
HEADS = 2


def _setup(N, delta, seed=0, n_rows=256):
    inp = I.make_inputs(1, HEADS, HEADS, N, D, delta=delta, seed=seed, descale="head")
    rows = np.sort(np.random.default_rng(1).choice(N, min(n_rows, N), replace=False))
    refs = []
    for h in range(HEADS):
        s, _ = A.head_logits_float(inp["q"][0, h], inp["k"][0, h], D, rows=rows)
        refs.append(A.exact_attention(s, inp["v"][0, h]))
    return inp, to_device(inp), rows, np.stack(refs)


def _mse(t, rows, ref, *, order, S, denominator="fp32"):
    o, _ = binding.fwd_ex(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=False, kv_order=order,
                          S=S, n_sink=4, denominator=denominator)
    torch.cuda.synchronize()
    got = o[0].cpu().numpy()[:, rows].astype(np.float64)
    return float(np.mean((got - ref) ** 2))


def test_gain_grows_with_sequence_length():
    ratios = []
    for N in (1024, 4096, 16384):
        say(f"case N={N} delta=7")
        _, t, rows, ref = _setup(N, 7.0)
        fwd1 = _mse(t, rows, ref, order="forward", S=1.0)
        rev256 = _mse(t, rows, ref, order="reverse", S=256.0)
        ratios.append(fwd1 / rev256)
        say(f"  N={N}: MSE forward S=1 {fwd1:.4e}  reverse S=256 {rev256:.4e}  ratio {ratios[-1]:.3f}")
    assert ratios[0] < ratios[1] < ratios[2]
    assert ratios[2] > 1.3


def test_power_of_two_wins_its_octave():
    _, t, rows, ref = _setup(4096, 7.0)
    say("case S sweep, forward, N=4096 delta=7")
    mse = {}
    for S in (1.0, 8.0, 12.0, 16.0, 24.0, 32.0, 48.0, 64.0, 96.0, 128.0, 192.0, 256.0, 320.0, 384.0, 448.0):
        mse[S] = _mse(t, rows, ref, order="forward", S=S)
        say(f"  S={S:6.1f}  MSE {mse[S]:.5e}")
    for k in (8.0, 16.0, 32.0, 64.0, 128.0):
        assert mse[k] < mse[1.5 * k], k
    assert mse[1.0] > max(v for s, v in mse.items() if s > 1.0)


@pytest.mark.parametrize("N", [4096, 16384])
def test_quantized_denominator(N):
    _, t, rows, ref = _setup(N, 7.0)
    say(f"case denominators, N={N} delta=7")
    r_fp32 = _mse(t, rows, ref, order="reverse", S=256.0)
    r_q = _mse(t, rows, ref, order="reverse", S=256.0, denominator="quantized")
    f_fp32 = _mse(t, rows, ref, order="forward", S=1.0)
    f_q = _mse(t, rows, ref, order="forward", S=1.0, denominator="quantized")
    say(f"  reverse S=256: fp32 {r_fp32:.4e} quantized {r_q:.4e} | forward S=1: fp32 {f_fp32:.4e} "
        f"quantized {f_q:.4e}")
    assert r_q <= 1.02 * r_fp32
    assert f_q > 10.0 * f_fp32


def test_sink_last_keeps_the_error_of_clean_inputs():
    _, t, rows, ref = _setup(4096, 10.0)
    say("case sink-last vs reverse, N=4096 delta=10")
    rev = _mse(t, rows, ref, order="reverse", S=256.0)
    last = _mse(t, rows, ref, order="reverse_sink_last", S=256.0)
    say(f"  reverse {rev:.5e}  sink-last {last:.5e}")
    assert abs(last / rev - 1.0) < 0.01


@pytest.mark.parametrize("delta", [7.0, 8.0, 10.0])
def test_s256_against_s384_and_s448(delta):
    """MSE of the P cast alone (against exact attention of the dequantized E4M3 operands,
    no cast) on the GPU path for S = 256, 384 and 448, forward order, 1024 rows of each of
    two heads. The gains of 384 and 448 over 256 must match the oracle's on the same rows
    (within 3 points); whether 256 wins is printed. With E4M3 Q, K, V the large P~ fall
    differently within an octave than with the pages' fp32 operands, and the oracle itself
    has 448 ahead at some Δ (the fp32-operand case, where 256 wins by 3-6%, is pinned on the
    CPU)."""
    N = 4096
    inp, t, rows, _ = _setup(N, delta, n_rows=1024)
    refs, heads = [], []
    for h in range(HEADS):
        s8, _ = A.head_logits_e4m3(inp["q8"][0, h], inp["k8"][0, h], inp["qd"][0, h], inp["kd"][0, h], D, rows=rows)
        vf = e4m3.decode(inp["v8"][0, h]) * float(inp["vd"][0, h])
        refs.append(A.exact_attention(s8, vf))
        heads.append((s8, vf))
    ref = np.stack(refs)
    say(f"case S=256 vs 384/448 (P-cast error), forward, N={N} delta={delta}")
    scales = (256.0, 384.0, 448.0)
    mse = {S: _mse(t, rows, ref, order="forward", S=S) for S in scales}
    mse_o = {}
    for S in scales:
        outs = [A.online_softmax_pcast(s8, vf, kv_order="forward", S=S)[0] for (s8, vf) in heads]
        mse_o[S] = float(np.mean((np.stack(outs) - ref) ** 2))
    gain = {S: mse[S] / mse[256.0] - 1.0 for S in scales[1:]}
    gain_o = {S: mse_o[S] / mse_o[256.0] - 1.0 for S in scales[1:]}
    say(f"  GPU MSE S=256 {mse[256.0]:.5e}  S=384 {100 * gain[384.0]:+.1f}%  S=448 {100 * gain[448.0]:+.1f}% | "
        f"oracle S=384 {100 * gain_o[384.0]:+.1f}%  S=448 {100 * gain_o[448.0]:+.1f}% | "
        f"S=256 lowest: {'yes' if min(gain.values()) > 0 else 'no'}")
    for S in scales[1:]:
        assert abs(gain[S] - gain_o[S]) <= 0.03, (S, gain[S], gain_o[S])
