"""GPU parity at sizes the oracle finishes in seconds: the HIP forward and collapse
count, called through the C ABI, against the fp64 oracle element by element.

Two references per case. (1) The pages' result: the oracle on the exact logits of the
decoded codes. The tolerance is 2e-3 plus an allowance derived from a bound on the FP8
matrix core's Q.K^T error (the stated truncation rule, evaluated as an interval per
query-key pair: never from running the model) and the fp32 band around E4M3 rounding
midpoints; the fraction of rows beyond 2e-3 and the largest deviation are printed and
held below fixed limits. (2) A secondary check: the oracle run on the logits the matrix
core forms (oracle.mfma_model), with only the fp32 band as allowance, which checks the
softmax, the cast and the block order without the logit error. Pair counts exact;
collapse counts within 0.5% (or the boundary-flagged pairs).
"""
import numpy as np
import pytest
import torch

from precision_attention_amd import inputs as I

from _gpu_util import check_both, gpu_counts, gpu_fwd, pair_counts, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("order", ["forward", "reverse"])
@pytest.mark.parametrize("S", [1.0, 16.0, 256.0, 448.0])
def test_tiny_noncausal_full_parity(order, S):
    w = I.WORKLOADS["tiny_noncausal_n1024_d64"]
    inp = I.make_workload_inputs(w, seed=0)
    t = to_device(inp)
    label = f"{w.name} {order} S={S}"
    say(f"case {label}")
    o = gpu_fwd(t, causal=False, order=order, S=S)
    c = gpu_counts(t, causal=False, order=order, S=S)
    check_both(inp, o, c, causal=False, order=order, S=S, label=label)


EDGE = [
    # B, H, Hkv, N, d, causal, order, S, delta
    (1, 1, 1, 64, 64, False, "forward", 256.0, 8.0),
    (1, 1, 1, 64, 128, True, "reverse", 256.0, 8.0),
    (1, 2, 1, 192, 128, True, "reverse", 448.0, 10.0),     # ragged query tile, GQA
    (1, 2, 2, 192, 128, False, "forward", 1.0, 6.0),
    (2, 4, 2, 320, 256, True, "reverse", 256.0, 12.0),
    (1, 3, 1, 128, 256, False, "forward", 16.0, 7.0),
    (2, 2, 2, 448, 64, True, "forward", 256.0, 8.0),
    (1, 8, 2, 256, 128, True, "forward", 1.0, 0.0),         # no sink at all
    (1, 1, 1, 512, 128, True, "reverse", 2.0, 4.0),
    (3, 2, 1, 640, 128, True, "reverse", 256.0, 10.0),
]


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,order,S,delta", EDGE)
def test_edge_shapes_full_parity(B, H, Hkv, N, d, causal, order, S, delta):
    inp = I.make_inputs(B, H, Hkv, N, d, delta=delta, seed=B * 100 + N, descale="head")
    t = to_device(inp)
    label = f"B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} {order} S={S} delta={delta}"
    say(f"case {label}")
    o = gpu_fwd(t, causal=causal, order=order, S=S)
    c = gpu_counts(t, causal=causal, order=order, S=S)
    check_both(inp, o, c, causal=causal, order=order, S=S, label=label)
    assert tuple(c[2:]) == pair_counts(B, H, N, causal)



def _random_configs(n=12, seed=2024):
    """Seeded random shapes and options, beyond the hand-picked edge cases: B, H, the
    grouped-query ratio, N (multiples of 64, not of 128 half the time), d, mask, order,
    S (powers of two and not) and the sink strength."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.integers(1, 3))
        H = Hkv * int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 3))
        N = 64 * int(rng.integers(1, 9 if d < 256 else 6))
        causal = bool(rng.integers(0, 2))
        order = str(rng.choice(["forward", "reverse"]))
        S = float(rng.choice([1.0, 2.0, 8.0, 64.0, 256.0, 3.0, 100.0, 448.0]))
        delta = float(rng.choice([0.0, 4.0, 8.0, 12.0]))
        out.append((B, H, Hkv, N, d, causal, order, S, delta))
    return out


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,order,S,delta", _random_configs())
def test_random_shapes_full_parity(B, H, Hkv, N, d, causal, order, S, delta):
    inp = I.make_inputs(B, H, Hkv, N, d, delta=delta, seed=7 * N + d + B, descale="head")
    t = to_device(inp)
    label = f"random B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} {order} S={S} delta={delta}"
    say(f"case {label}")
    o = gpu_fwd(t, causal=causal, order=order, S=S)
    c = gpu_counts(t, causal=causal, order=order, S=S)
    check_both(inp, o, c, causal=causal, order=order, S=S, label=label)
    assert tuple(c[2:]) == pair_counts(B, H, N, causal)

def test_literal_sink_construction():
    inp = I.make_inputs(1, 2, 1, 512, 128, delta=10.0, seed=3, descale="head", construction="literal")
    t = to_device(inp)
    for order in ("forward", "reverse"):
        say(f"case literal sinks N512 d128 {order}")
        o = gpu_fwd(t, causal=True, order=order, S=256.0)
        c = gpu_counts(t, causal=True, order=order, S=256.0)
        check_both(inp, o, c, causal=True, order=order, S=256.0, label=f"literal {order}")


@pytest.mark.parametrize("delta,order,S", [(0.0, "forward", 1.0), (7.0, "forward", 1.0), (7.0, "reverse", 256.0),
                                           (10.0, "forward", 16.0), (10.0, "reverse", 448.0),
                                           (12.0, "forward", 256.0), (12.0, "reverse", 256.0)])
def test_delta_sweep_one_head(delta, order, S):
    """Δ sweep shape (N = 4096, d = 128, non-causal, per-tensor descale): one head of
    the GPU run compared in full with the oracle."""
    w = I.WORKLOADS["sweep_noncausal_h8_n4096_d128"]
    inp = I.make_inputs(1, 2, 2, w.N, w.d, delta=delta, seed=0, descale="tensor", keep_float=False)
    t = to_device(inp)
    label = f"sweep delta={delta} {order} S={S}"
    say(f"case {label}")
    o = gpu_fwd(t, causal=False, order=order, S=S)
    one = {k: v[:, :1].contiguous() for k, v in t.items()}
    c = gpu_counts(one, causal=False, order=order, S=S)
    check_both(inp, o, c, causal=False, order=order, S=S, label=label, heads=[(0, 1)], count_heads=[(0, 0)])


def test_deterministic_bitwise():
    inp = I.make_inputs(1, 4, 2, 1024, 128, delta=8.0, seed=5, descale="head", keep_float=False)
    t = to_device(inp)
    say("case determinism N1024 d128 causal reverse")
    a = gpu_fwd(t, causal=True, order="reverse", S=256.0).clone()
    b = gpu_fwd(t, causal=True, order="reverse", S=256.0)
    assert torch.equal(a, b)


def test_float8_dtype_and_stream():
    inp = I.make_inputs(1, 1, 1, 256, 64, delta=8.0, seed=6, descale="tensor", keep_float=False)
    t = to_device(inp)
    say("case float8_e4m3fn view + side stream")
    ref = gpu_fwd(t, causal=True, order="reverse", S=256.0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        f8 = {k: (v.view(torch.float8_e4m3fn) if v.dtype == torch.uint8 else v) for k, v in t.items()}
        from precision_attention_amd import binding
        o = binding.fwd(f8["q8"], f8["k8"], f8["v8"], f8["qd"], f8["kd"], f8["vd"], causal=True,
                        kv_order="reverse", S=256.0)
    s.synchronize()
    assert torch.equal(o, ref)


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,order,S", [
    (1, 4, 2, 1024, 128, True, "reverse", 256.0), (2, 2, 2, 640, 64, False, "forward", 1.0),
    (1, 2, 1, 384, 256, True, "forward", 448.0)])
def test_fused_equals_separate(B, H, Hkv, N, d, causal, order, S):
    """fp8_attn_fwd_counted writes the same O (bitwise) as fp8_attn_fwd and the same
    counts as fp8_attn_p_collapse_count."""
    from precision_attention_amd import binding

    inp = I.make_inputs(B, H, Hkv, N, d, delta=10.0, seed=7, descale="head", keep_float=False)
    t = to_device(inp)
    say(f"case fused B{B} H{H} N{N} d{d} causal={causal} {order} S={S}")
    o = gpu_fwd(t, causal=causal, order=order, S=S)
    c = gpu_counts(t, causal=causal, order=order, S=S)
    of, cf = binding.fwd_counted(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=causal,
                                 kv_order=order, S=S, n_sink=4)
    torch.cuda.synchronize()
    assert torch.equal(o, of)
    assert np.array_equal(c, cf.cpu().numpy())
