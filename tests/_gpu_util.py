"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI binding
and compare with the CPU oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

from oracle import attention as oracle_attention
from precision_attention_amd import binding

O_TOL = 2e-3          # max-abs on unit-scale O (plus the rounding-boundary allowance)
COUNT_REL_TOL = 0.005  # collapse count: 0.5% relative (or the boundary-flagged pairs)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda:0")


def to_device(inp, keys=("q8", "k8", "v8", "qd", "kd", "vd")):
    dev = device()
    return {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev) for k in keys}


def gpu_fwd(t, *, causal, order, S):
    o = binding.fwd(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=causal, kv_order=order, S=S)
    torch.cuda.synchronize()
    return o


def gpu_counts(t, *, causal, order, S, n_sink=4):
    c = binding.p_collapse_count(t["q8"], t["k8"], t["qd"], t["kd"], causal=causal, kv_order=order,
                                 S=S, n_sink=n_sink)
    torch.cuda.synchronize()
    return c.cpu().numpy().astype(np.int64)


def oracle(inp, *, causal, order, S, rows=None, heads=None, counts=False, n_sink=4, logits="device",
           denominator="fp32"):
    return oracle_attention.attention_e4m3(inp["q8"], inp["k8"], inp["v8"], inp["qd"], inp["kd"], inp["vd"],
                                           causal=causal, kv_order=order, S=S, rows=rows, heads=heads,
                                           n_sink=n_sink, logits=logits, with_allowance=True,
                                           with_counts=counts, denominator=denominator)


def check_output(o_gpu, ref, label=""):
    """o_gpu: full [B,H,N,d] device tensor; ref: oracle dict (heads x rows)."""
    got = np.stack([o_gpu[b, h].cpu().numpy()[ref["rows"]] for (b, h) in ref["heads"]])
    diff = np.abs(got - ref["o"])
    excess = diff - (O_TOL + ref["allow"])
    rows_allow = int(((diff > O_TOL).any(axis=2)).sum())
    say(f"  {label}: max|dO| {diff.max():.3g}  rows beyond {O_TOL} (inside their allowance) {rows_allow}"
        f" of {diff.shape[0] * diff.shape[1]}")
    assert np.isfinite(got).all(), "non-finite output"
    assert excess.max() <= 0, f"{label}: output exceeds tolerance by {excess.max():.3g}"
    return diff.max()


def check_counts(c_gpu, c_ref, zero_flagged, label=""):
    say(f"  {label}: counts gpu {list(c_gpu)} oracle {list(c_ref)} (boundary-flagged {zero_flagged})")
    assert c_gpu[2] == c_ref[2] and c_gpu[3] == c_ref[3], "pair counts differ"
    for i in (0, 1):
        slack = max(COUNT_REL_TOL * c_ref[i], zero_flagged)
        assert abs(int(c_gpu[i]) - int(c_ref[i])) <= slack, f"count[{i}] differs"


def check_both(inp, o, c, *, causal, order, S, label, rows=None, heads=None, count_heads=None, n_sink=4,
               denominator="fp32"):
    """Tight check against the oracle on the device's matrix-core logits, then the check
    against the exact-logit oracle with its wider (matrix-core aware) tolerance."""
    opts = {"n_sink": n_sink, "denominator": denominator}
    for logits in ("device", "exact"):
        ref = oracle(inp, causal=causal, order=order, S=S, rows=rows, heads=heads, logits=logits,
                     counts=c is not None and count_heads is None, **opts)
        check_output(o, ref, f"{label} [{logits} logits]")
        if c is not None:
            cref = ref if count_heads is None else oracle(inp, causal=causal, order=order, S=S, heads=count_heads,
                                                          logits=logits, counts=True, **opts)
            check_counts(c, cref["counts"], cref["zero_flagged"], f"{label} [{logits} logits]")


def pair_counts(B, H, N, causal, n_sink=4, block=64):
    """Unmasked non-sink (i, j) pairs, total and inside blocks holding a sink key."""
    i = np.arange(N, dtype=np.int64)
    sink_block_end = ((n_sink + block - 1) // block) * block     # keys [0, end) lie in sink blocks
    if causal:
        tot = np.maximum(0, i - n_sink + 1).sum()
        sb = np.maximum(0, np.minimum(i, sink_block_end - 1) - n_sink + 1).sum()
    else:
        tot = N * max(0, N - n_sink)
        sb = N * max(0, sink_block_end - n_sink)
    return int(B * H * tot), int(B * H * sb)
