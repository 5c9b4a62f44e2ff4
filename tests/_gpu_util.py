"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI binding
and compare with the CPU oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

from oracle import attention as oracle_attention
from precision_attention_amd import binding

O_TOL = 2e-3          # max-abs on unit-scale O (plus the allowance of the reference)
COUNT_REL_TOL = 0.005  # collapse count: 0.5% relative (or the boundary-flagged pairs)
# Against the exact-logit oracle (the pages' result), beside the element-wise tolerance:
# the fraction of checked rows whose deviation exceeds O_TOL anywhere, and the largest
# deviation. Both stem from the logit error of Q.K^T and from P·S values next to an E4M3
# rounding midpoint (a sink's code moving one E4M3 step, at most 1/8 of its value, moves
# its row by up to ~0.25 with heavy-tailed V).
ROWS_BEYOND_LIMIT = {"e4m3_mfma": 0.05, "fp32": 0.01}
MAX_DEV_LIMIT = 0.5


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


def oracle(inp, *, causal, order, S, rows=None, heads=None, counts=False, n_sink=4, logits="exact",
           denominator="fp32", qk="e4m3_mfma"):
    return oracle_attention.attention_e4m3(inp["q8"], inp["k8"], inp["v8"], inp["qd"], inp["kd"], inp["vd"],
                                           causal=causal, kv_order=order, S=S, rows=rows, heads=heads,
                                           n_sink=n_sink, logits=logits, with_allowance=True,
                                           with_counts=counts, denominator=denominator, qk_accumulation=qk)


def s_on_a_midpoint(S):
    """True if S lies within the fp32 band of an E4M3 rounding midpoint: then every row's
    maximum (P~ = 1, cast S) is a legitimate tie that the device may round either way, and
    the fraction of rows beyond O_TOL says nothing (S = 100 lies between 96 and 104)."""
    from oracle import e4m3

    vals = e4m3.all_finite_values()
    mids = (vals[:-1] + vals[1:]) / 2.0
    return bool((np.abs(S - mids) <= oracle_attention.FLIP_REL_WINDOW * mids).any())


def check_output(o_gpu, ref, label="", qk=None, S=None):
    """o_gpu: full [B,H,N,d] device tensor; ref: oracle dict (heads x rows). Every element
    within O_TOL plus its allowance; with ``qk`` (an exact-logit reference) also the row
    fraction beyond O_TOL (unless S sits on a midpoint) and the largest deviation within
    their limits."""
    got = np.stack([o_gpu[b, h].cpu().numpy()[ref["rows"]] for (b, h) in ref["heads"]])
    diff = np.abs(got - ref["o"])
    excess = diff - (O_TOL + ref["allow"])
    beyond = (diff > O_TOL).any(axis=2)
    n_rows = diff.shape[0] * diff.shape[1]
    say(f"  {label}: max|dO| {diff.max():.3g}; rows beyond {O_TOL}: {int(beyond.sum())} of {n_rows} "
        f"({beyond.mean():.4f}); worst excess over tolerance {excess.max():.3g}")
    assert np.isfinite(got).all(), "non-finite output"
    assert excess.max() <= 0, f"{label}: output exceeds tolerance by {excess.max():.3g}"
    if qk is not None:
        if S is not None and s_on_a_midpoint(S):
            say(f"  (S = {S} lies on an E4M3 rounding midpoint: every row maximum is a tie; no row-fraction limit)")
        else:
            assert beyond.mean() <= ROWS_BEYOND_LIMIT[qk], f"{label}: {beyond.mean():.4f} of rows beyond {O_TOL}"
        assert diff.max() <= MAX_DEV_LIMIT, f"{label}: max|dO| {diff.max():.3g}"
    return diff.max()


def check_counts(c_gpu, c_ref, zero_flagged, label=""):
    say(f"  {label}: counts gpu {list(c_gpu)} oracle {list(c_ref)} (boundary-flagged {zero_flagged})")
    assert c_gpu[2] == c_ref[2] and c_gpu[3] == c_ref[3], "pair counts differ"
    for i in (0, 1):
        slack = max(COUNT_REL_TOL * c_ref[i], zero_flagged)
        assert abs(int(c_gpu[i]) - int(c_ref[i])) <= slack, f"count[{i}] differs"


def check_both(inp, o, c, *, causal, order, S, label, rows=None, heads=None, count_heads=None, n_sink=4,
               denominator="fp32", qk="e4m3_mfma"):
    """The check against the pages' result first: the exact-logit oracle, with the
    tolerance that the logit interval of the device's Q.K^T accumulation ``qk`` implies
    (analytic, from the stated accumulation rule) and limits on the rows beyond O_TOL.
    Then, for the FP8 matrix-core path, the secondary check against the oracle run on the
    matrix core's own logits with only the fp32 band as allowance (softmax, cast and
    block order checked without the logit error)."""
    opts = {"n_sink": n_sink, "denominator": denominator, "qk": qk}
    refs = [("exact", True)] + ([("device", False)] if qk == "e4m3_mfma" else [])
    for logits, primary in refs:
        ref = oracle(inp, causal=causal, order=order, S=S, rows=rows, heads=heads, logits=logits,
                     counts=c is not None and count_heads is None, **opts)
        check_output(o, ref, f"{label} [{logits} logits]", qk=qk if primary else None, S=S)
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
