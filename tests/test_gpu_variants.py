"""GPU parity of the two options of fp8_attn_fwd_ex against the oracle: the sink-last
reverse schedule (block 0's non-sink keys visited before the sink tokens) and the
quantized row-sum denominator. Same two-reference check as the main parity tests
(exact-logit oracle with the analytic logit-interval allowance, then the device-logit
oracle with the fp32 band only); pair counts exact, collapse counts within 0.5% or the
boundary-flagged pairs."""
import numpy as np
import pytest
import torch

from precision_attention_amd import binding
from precision_attention_amd import inputs as I

from _gpu_util import check_both, pair_counts, say, to_device

pytestmark = pytest.mark.gpu


def _run(t, *, causal, order, S, n_sink, denominator):
    o, c = binding.fwd_ex(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=causal, kv_order=order,
                          S=S, n_sink=n_sink, denominator=denominator, count=True)
    torch.cuda.synchronize()
    return o, c.cpu().numpy().astype(np.int64)


CASES = [
    # B, H, Hkv, N, d, causal, order, S, delta, n_sink, denominator
    (1, 1, 1, 1024, 64, False, "reverse_sink_last", 256.0, 10.0, 4, "fp32"),
    (1, 1, 1, 1024, 64, False, "reverse_sink_last", 1.0, 8.0, 4, "quantized"),
    (1, 2, 1, 192, 128, True, "reverse_sink_last", 256.0, 12.0, 4, "fp32"),      # ragged tile, GQA
    (1, 1, 1, 64, 128, True, "reverse_sink_last", 256.0, 10.0, 4, "fp32"),       # one block only
    (2, 2, 2, 320, 256, True, "reverse_sink_last", 448.0, 10.0, 1, "quantized"),
    (1, 2, 2, 256, 128, True, "reverse_sink_last", 16.0, 8.0, 64, "fp32"),       # block 0 all sinks
    (1, 2, 2, 256, 128, False, "reverse_sink_last", 256.0, 8.0, 0, "fp32"),      # no split
    (1, 2, 1, 512, 128, True, "forward", 256.0, 10.0, 4, "quantized"),
    (1, 2, 1, 512, 128, True, "reverse", 448.0, 10.0, 4, "quantized"),
    (1, 4, 2, 384, 64, False, "forward", 1.0, 6.0, 4, "quantized"),
]


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,order,S,delta,n_sink,denominator", CASES)
def test_variant_parity(B, H, Hkv, N, d, causal, order, S, delta, n_sink, denominator):
    inp = I.make_inputs(B, H, Hkv, N, d, delta=delta, seed=7 * N + d, descale="head")
    t = to_device(inp)
    label = f"B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} {order} S={S} n_sink={n_sink} {denominator}"
    say(f"case {label}")
    o, c = _run(t, causal=causal, order=order, S=S, n_sink=n_sink, denominator=denominator)
    check_both(inp, o, c, causal=causal, order=order, S=S, label=label, n_sink=n_sink, denominator=denominator)
    assert tuple(c[2:]) == pair_counts(B, H, N, causal, n_sink=n_sink)



def _random_cases(n=10, seed=77):
    """Seeded random shapes with the fwd_ex options: the three orders, both denominators,
    n_sink from 0 to 64 (0 to N for the plain orders), S powers of two and not."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.integers(1, 3))
        H = Hkv * int(rng.choice([1, 2]))
        N = 64 * int(rng.integers(1, 7 if d < 256 else 5))
        causal = bool(rng.integers(0, 2))
        order = str(rng.choice(["forward", "reverse", "reverse_sink_last"]))
        S = float(rng.choice([1.0, 16.0, 256.0, 5.0, 448.0]))
        delta = float(rng.choice([0.0, 8.0, 12.0]))
        n_sink = int(rng.choice([0, 1, 4, 17, 64]))
        denominator = str(rng.choice(["fp32", "quantized"]))
        out.append((1, H, Hkv, N, d, causal, order, S, delta, n_sink, denominator))
    return out


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,order,S,delta,n_sink,denominator", _random_cases())
def test_variant_random_parity(B, H, Hkv, N, d, causal, order, S, delta, n_sink, denominator):
    test_variant_parity(B, H, Hkv, N, d, causal, order, S, delta, n_sink, denominator)

def test_sink_last_has_no_collapse_on_clean_sinks():
    """What the schedule is for, on the GPU: clean sinks at Δ = 10, S = 256, N = 4096;
    plain reverse collapses part of block 0's non-sink keys, sink-last none at all."""
    inp = I.make_inputs(1, 4, 4, 4096, 128, delta=10.0, seed=0, descale="tensor", keep_float=False)
    t = to_device(inp)
    say("case sink-last vs reverse, N4096 d128 delta 10")
    _, c_rev = _run(t, causal=False, order="reverse", S=256.0, n_sink=4, denominator="fp32")
    _, c_last = _run(t, causal=False, order="reverse_sink_last", S=256.0, n_sink=4, denominator="fp32")
    say(f"  reverse {list(c_rev)}  sink-last {list(c_last)}")
    assert c_rev[1] > 0 and c_rev[0] == c_rev[1]
    assert c_last[0] == 0
    assert list(c_last[2:]) == list(c_rev[2:])


@pytest.mark.parametrize("order", ["forward", "reverse"])
def test_ex_defaults_equal_the_plain_entry_points(order):
    """fwd_ex with the pages' two orders and the fp32 denominator runs the same kernel as
    fp8_attn_fwd / fp8_attn_fwd_counted: bitwise equal outputs and counts."""
    inp = I.make_inputs(1, 4, 2, 640, 128, delta=10.0, seed=5, descale="head", keep_float=False)
    t = to_device(inp)
    say(f"case ex vs plain, {order}")
    o_ex, c_ex = _run(t, causal=True, order=order, S=256.0, n_sink=4, denominator="fp32")
    o_pl = binding.fwd(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=True, kv_order=order, S=256.0)
    o_ct, c_ct = binding.fwd_counted(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=True,
                                     kv_order=order, S=256.0, n_sink=4)
    o_nc, c_nc = binding.fwd_ex(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=True,
                                kv_order=order, S=256.0)
    torch.cuda.synchronize()
    assert c_nc is None
    assert torch.equal(o_ex, o_pl) and torch.equal(o_ex, o_ct) and torch.equal(o_ex, o_nc)
    assert list(c_ex) == list(c_ct.cpu().numpy())
