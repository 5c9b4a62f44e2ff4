"""GPU parity of the exact-Q.K^T forward (fp8_attn_fwd_exact_qk) against the oracle on
exact logits: Q.K^T from exact E4M3 products accumulated in fp32 (bf16 matrix cores), so
the only logit error is fp32 accumulation rounding (oracle.mfma_model.fp32_accumulation_bound,
one rounding per 16-slot instruction) and the only allowance beyond 2e-3 is the fp32 band
around E4M3 rounding midpoints that this implies. This is the pages' computation (P-Cast
technical summary, section 1: only P is cast) without the FP8 matrix core's truncation.
Pair counts exact, collapse counts within 0.5% (or the boundary-flagged pairs)."""
import numpy as np
import pytest
import torch

from precision_attention_amd import binding
from precision_attention_amd import inputs as I

from _gpu_util import check_both, check_output, oracle, pair_counts, say, to_device

pytestmark = pytest.mark.gpu


def _run(t, *, causal, order, S, n_sink=4, denominator="fp32", count=True):
    o, c = binding.fwd_exact_qk(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=causal,
                                kv_order=order, S=S, n_sink=n_sink, denominator=denominator, count=count)
    torch.cuda.synchronize()
    return o, (None if c is None else c.cpu().numpy().astype(np.int64))


@pytest.mark.parametrize("order", ["forward", "reverse"])
@pytest.mark.parametrize("S", [1.0, 256.0, 448.0])
def test_tiny_noncausal(order, S):
    w = I.WORKLOADS["tiny_noncausal_n1024_d64"]
    inp = I.make_workload_inputs(w, seed=0)
    t = to_device(inp)
    label = f"exact-qk {w.name} {order} S={S}"
    say(f"case {label}")
    o, c = _run(t, causal=False, order=order, S=S)
    check_both(inp, o, c, causal=False, order=order, S=S, label=label, qk="fp32")


CASES = [
    # B, H, Hkv, N, d, causal, order, S, delta, n_sink, denominator
    (1, 1, 1, 64, 128, True, "reverse", 256.0, 8.0, 4, "fp32"),
    (1, 2, 1, 192, 128, True, "reverse", 448.0, 10.0, 4, "fp32"),         # ragged tile, GQA
    (1, 2, 2, 192, 128, False, "forward", 1.0, 6.0, 4, "fp32"),
    (2, 2, 2, 448, 64, True, "forward", 256.0, 8.0, 4, "fp32"),
    (1, 8, 2, 256, 128, True, "forward", 1.0, 0.0, 4, "fp32"),            # no sink
    (3, 2, 1, 640, 128, True, "reverse", 256.0, 10.0, 4, "fp32"),
    (1, 1, 1, 1024, 64, False, "reverse_sink_last", 256.0, 10.0, 4, "fp32"),
    (1, 2, 1, 512, 128, True, "reverse", 448.0, 10.0, 4, "quantized"),
    (1, 2, 2, 256, 128, True, "reverse_sink_last", 16.0, 8.0, 64, "fp32"),
    (1, 4, 2, 384, 64, False, "forward", 3.0, 6.0, 4, "quantized"),       # S not a power of two
]


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,order,S,delta,n_sink,denominator", CASES)
def test_shapes_and_options(B, H, Hkv, N, d, causal, order, S, delta, n_sink, denominator):
    inp = I.make_inputs(B, H, Hkv, N, d, delta=delta, seed=11 * N + d + B, descale="head")
    t = to_device(inp)
    label = f"exact-qk B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} {order} S={S} n_sink={n_sink} {denominator}"
    say(f"case {label}")
    o, c = _run(t, causal=causal, order=order, S=S, n_sink=n_sink, denominator=denominator)
    check_both(inp, o, c, causal=causal, order=order, S=S, label=label, n_sink=n_sink, denominator=denominator,
               qk="fp32")
    assert tuple(c[2:]) == pair_counts(B, H, N, causal, n_sink=n_sink)


@pytest.mark.parametrize("delta,order,S", [(7.0, "forward", 1.0), (10.0, "reverse", 256.0), (12.0, "forward", 448.0)])
def test_delta_sweep_one_head(delta, order, S):
    inp = I.make_inputs(1, 1, 1, 4096, 128, delta=delta, seed=0, descale="tensor", keep_float=False)
    t = to_device(inp)
    label = f"exact-qk sweep delta={delta} {order} S={S}"
    say(f"case {label}")
    o, c = _run(t, causal=False, order=order, S=S)
    check_both(inp, o, c, causal=False, order=order, S=S, label=label, qk="fp32")


def test_gqa_causal_n32768_sampled_rows():
    """The benchmark workload (B=1, 32 query / 8 KV heads, N = 32768, d = 128, causal,
    reverse, S = 256) on sampled rows of three heads, with the pre-sink collapse count
    exactly zero; also the output distance to the FP8-matrix-core forward (the effect of
    that instruction's truncation, printed)."""
    w = I.WORKLOADS["gqa_causal_h32_kv8_n32768_d128"]
    inp = I.make_workload_inputs(w, seed=0, keep_float=False)
    t = to_device(inp)
    label = f"exact-qk {w.name} reverse S=256"
    say(f"case {label}")
    o, c = _run(t, causal=True, order="reverse", S=256.0)
    rows = I.sample_rows(w.N, 320, seed=0)
    ref = oracle(inp, causal=True, order="reverse", S=256.0, rows=rows, heads=[(0, 0), (0, 5), (0, 31)], qk="fp32")
    check_output(o, ref, f"{label} [exact logits]", qk="fp32")
    tot, sink = pair_counts(w.B, w.H, w.N, w.causal)
    assert (int(c[2]), int(c[3])) == (tot, sink)
    assert int(c[0]) - int(c[1]) == 0
    o_fast = binding.fwd(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=True, kv_order="reverse", S=256.0)
    torch.cuda.synchronize()
    d = (o_fast - o).abs()
    say(f"  counts {list(c)}; FP8-matrix-core forward vs exact-Q.K^T forward: max|dO| {float(d.max()):.3g}, "
        f"rows beyond 2e-3 {float((d.amax(dim=3) > 2e-3).float().mean()):.4f}")


def test_deterministic_and_workspace_reuse():
    inp = I.make_inputs(1, 4, 2, 1024, 128, delta=8.0, seed=5, descale="head", keep_float=False)
    t = to_device(inp)
    say("case exact-qk determinism")
    need = binding.load().fp8_attn_fwd_exact_qk_workspace_bytes(1, 2, 1024, 128)
    ws = torch.empty(need, dtype=torch.uint8, device=t["q8"].device)
    a, _ = binding.fwd_exact_qk(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=True, workspace=ws)
    a = a.clone()
    b, _ = binding.fwd_exact_qk(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(ValueError):
        binding.fwd_exact_qk(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=True,
                             workspace=torch.empty(need - 16, dtype=torch.uint8, device=t["q8"].device))
