"""GPU parity over a seeded random sweep that crosses the forward entry points with the
options and shapes: fp8_attn_fwd_counted (which picks the 16- or 32-row kernel),
fp8_attn_fwd_ex and fp8_attn_fwd_exact_qk; batch, head grouping, every head size, ragged
query tiles, both masks, the three block orders, S powers of two and not, sink strength,
both sink constructions, n_sink and both denominators. Every case is checked against the
exact-logit oracle (with the allowance its Q.K^T accumulation implies) and the counts
against the oracle's and the closed-form pair totals. FP8ATTN_SWEEP_CASES and
FP8ATTN_SWEEP_SEED widen or reseed the sweep (default: 24 cases, seed 4242)."""
import os

import numpy as np
import pytest
import torch

from precision_attention_amd import binding
from precision_attention_amd import inputs as I

from _gpu_util import check_both, pair_counts, say, to_device

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        entry = ("counted", "ex", "exact_qk")[i % 3]
        d = int(rng.choice([64, 128] if entry == "exact_qk" else [64, 128, 128, 256]))
        B = int(rng.choice([1, 1, 2, 3]))
        Hkv = int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2, 4]))
        N = 64 * int(rng.integers(1, 13 if d < 256 else 7))
        causal = bool(rng.integers(0, 2))
        orders = ["forward", "reverse"] + ([] if entry == "counted" else ["reverse_sink_last"])
        order = str(rng.choice(orders))
        S = float(rng.choice([1.0, 2.0, 16.0, 5.0, 256.0, 448.0]))
        delta = float(rng.choice([0.0, 6.0, 8.0, 10.0, 12.0]))
        construction = str(rng.choice(["clean", "literal"]))
        n_sink = int(rng.choice([0, 1, 4, 17, 64]))
        n_sink = min(n_sink, N)
        denominator = "fp32" if entry == "counted" else str(rng.choice(["fp32", "quantized"]))
        out.append((entry, B, H, Hkv, N, d, causal, order, S, delta, construction, n_sink, denominator))
    return out


@pytest.mark.parametrize("entry,B,H,Hkv,N,d,causal,order,S,delta,construction,n_sink,denominator",
                         _cases(n=int(os.environ.get("FP8ATTN_SWEEP_CASES", "24")),
                                seed=int(os.environ.get("FP8ATTN_SWEEP_SEED", "4242"))))
def test_random_sweep(entry, B, H, Hkv, N, d, causal, order, S, delta, construction, n_sink, denominator):
    inp = I.make_inputs(B, H, Hkv, N, d, delta=delta, seed=13 * N + d + B + H, descale="head",
                        construction=construction)
    t = to_device(inp)
    label = (f"sweep {entry} B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} {order} S={S} delta={delta} "
             f"{construction} n_sink={n_sink} {denominator}")
    say(f"case {label}")
    args = (t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"])
    if entry == "counted":
        o, c = binding.fwd_counted(*args, causal=causal, kv_order=order, S=S, n_sink=n_sink)
    elif entry == "ex":
        o, c = binding.fwd_ex(*args, causal=causal, kv_order=order, S=S, n_sink=n_sink, denominator=denominator,
                              count=True)
    else:
        o, c = binding.fwd_exact_qk(*args, causal=causal, kv_order=order, S=S, n_sink=n_sink,
                                    denominator=denominator, count=True)
    torch.cuda.synchronize()
    c = c.cpu().numpy().astype(np.int64)
    check_both(inp, o, c, causal=causal, order=order, S=S, label=label, n_sink=n_sink,
               denominator=denominator, qk="fp32" if entry == "exact_qk" else "e4m3_mfma")
    assert tuple(c[2:]) == pair_counts(B, H, N, causal, n_sink=n_sink)
