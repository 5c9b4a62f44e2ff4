"""GPU parity on the method's degenerate inputs, each against the exact-logit oracle and a
closed form:
- Q = 0: every logit is 0, so every P~ is 1 and casts exactly to the code of S; O is the
  mean of the decoded V over the keys a row sees (the prefix mean when causal), and no P
  collapses;
- V = 0: O is exactly 0, whatever the scores;
- sharp logits (logits 64 times sharper, on the exact Q.K^T entry point): each row's softmax
  is nearly one-hot and almost every non-maximal P collapses.
Shapes run on both forward kernels (16 and 32 rows per wave) and d = 64 and 128."""
import numpy as np
import pytest
import torch

from oracle import e4m3
from precision_attention_amd import binding
from precision_attention_amd import inputs as I

from _gpu_util import O_TOL, check_both, pair_counts, say, to_device

pytestmark = pytest.mark.gpu

SHAPES = [
    # B, H, Hkv, N, d, causal, order
    (1, 2, 1, 448, 128, True, "reverse"),      # small causal grid: two walk groups
    (1, 2, 2, 320, 64, False, "forward"),      # d = 64: 32-row waves
    (2, 4, 2, 256, 128, False, "reverse"),
]


def _run(inp, causal, order, S=256.0):
    t = to_device(inp)
    o, c = binding.fwd_counted(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=causal,
                               kv_order=order, S=S, n_sink=4)
    torch.cuda.synchronize()
    return o, c.cpu().numpy().astype(np.int64)


def _decoded_v(inp):
    """Decoded V [B, Hkv, N, d] in fp64 (value = code value * descale)."""
    v = e4m3.decode(inp["v8"]).astype(np.float64)
    return v * inp["vd"].astype(np.float64)[:, :, None, None]


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,order", SHAPES)
def test_zero_queries_give_the_mean_of_v(B, H, Hkv, N, d, causal, order):
    inp = I.make_inputs(B, H, Hkv, N, d, delta=8.0, seed=N + d, descale="head")
    inp["q8"][...] = 0
    label = f"Q=0 B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} {order}"
    say(f"case {label}")
    o, c = _run(inp, causal, order)
    check_both(inp, o, c, causal=causal, order=order, S=256.0, label=label)
    v = _decoded_v(inp)
    G = H // Hkv
    got = o.cpu().numpy()
    for b in range(B):
        for h in range(H):
            vk = v[b, h // G]
            ref = np.cumsum(vk, axis=0) / np.arange(1, N + 1)[:, None] if causal else np.broadcast_to(vk.mean(0), vk.shape)
            assert np.abs(got[b, h] - ref).max() <= O_TOL, f"{label}: head {h} differs from the mean of V"
    assert c[0] == 0 and c[1] == 0
    assert (int(c[2]), int(c[3])) == pair_counts(B, H, N, causal)


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,order", SHAPES)
def test_zero_values_give_zero_output(B, H, Hkv, N, d, causal, order):
    inp = I.make_inputs(B, H, Hkv, N, d, delta=10.0, seed=2 * N + d, descale="head")
    inp["v8"][...] = 0
    label = f"V=0 B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} {order}"
    say(f"case {label}")
    o, c = _run(inp, causal, order)
    assert torch.count_nonzero(o).item() == 0
    check_both(inp, o, c, causal=causal, order=order, S=256.0, label=label)


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,order", SHAPES)
def test_sharp_logits_nearly_one_hot(B, H, Hkv, N, d, causal, order):
    """Logits 64 times sharper than the workloads' (Q and K descales x 8): the softmax is
    nearly one-hot and almost every non-sink P collapses. Run on the exact Q.K^T entry point:
    the FP8 matrix core's logit error grows with the logit scale, and at this sharpness its
    analytic allowance would leave too little of the check."""
    inp = I.make_inputs(B, H, Hkv, N, d, delta=8.0, seed=3 * N + d, descale="head")
    inp["qd"] = (inp["qd"] * 8.0).astype(np.float32)
    inp["kd"] = (inp["kd"] * 8.0).astype(np.float32)
    label = f"sharp logits B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} {order}"
    say(f"case {label}")
    t = to_device(inp)
    o, c = binding.fwd_exact_qk(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=causal, kv_order=order,
                                S=256.0, n_sink=4, denominator="fp32", count=True)
    torch.cuda.synchronize()
    c = c.cpu().numpy().astype(np.int64)
    check_both(inp, o, c, causal=causal, order=order, S=256.0, label=label, qk="fp32")
    tot, sink = pair_counts(B, H, N, causal)
    assert (int(c[2]), int(c[3])) == (tot, sink)
    frac = int(c[0]) / tot
    say(f"  collapsed fraction of non-sink pairs {frac:.4f}")
    assert frac > 0.95
