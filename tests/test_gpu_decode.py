"""GPU parity of the split-KV decode (fp8_attn_decode) against the oracle's decode:
one query row per head (drawn like any query row, so the sink construction applies),
every query over all N keys, the split partition reproduced by
the oracle. Same two references as the prefill parity tests: the exact-logit oracle with
the analytic logit-interval allowance, and the oracle on the matrix core's own logits with
only the rounding-boundary allowance."""
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from precision_attention_amd import binding
from precision_attention_amd import inputs as I

from _gpu_util import MAX_DEV_LIMIT, O_TOL, ROWS_BEYOND_LIMIT, say, to_device

pytestmark = pytest.mark.gpu


def _decode_inputs(B, H, Hkv, N, d, delta, seed, descale="head"):
    inp = I.make_inputs(B, H, Hkv, N, d, delta=delta, seed=seed, descale=descale, keep_float=False, n_q=1)
    inp["q8"] = np.ascontiguousarray(inp["q8"][:, :, 0, :])        # q [B, H, d]
    return inp


def _check(inp, o_gpu, *, order, S, n_split, label, heads=None):
    """Exact-logit oracle with the analytic logit interval (primary; also the row fraction
    beyond O_TOL and the largest deviation within their limits), then the oracle on the
    matrix core's own logits with the fp32 band only."""
    got = o_gpu.cpu().numpy()
    for logits in ("exact", "device"):
        ref = A.decode_e4m3(inp["q8"], inp["k8"], inp["v8"], inp["qd"], inp["kd"], inp["vd"], kv_order=order, S=S,
                            n_split=n_split, logits=logits, with_allowance=True, heads=heads)
        sel = [(b, h) for b in range(got.shape[0]) for h in range(got.shape[1])] if heads is None else heads
        idx = tuple(np.array(sel).T)
        diff = np.abs(got[idx] - ref["o"][idx])
        excess = diff - (O_TOL + ref["allow"][idx])
        beyond = (diff > O_TOL).any(axis=1)
        say(f"  {label} [{logits} logits]: max|dO| {diff.max():.3g}; rows beyond {O_TOL}: {int(beyond.sum())} "
            f"of {len(sel)}; worst excess {excess.max():.3g}")
        assert np.isfinite(got).all()
        assert excess.max() <= 0, f"{label}: exceeds tolerance by {excess.max():.3g}"
        if logits == "exact":
            assert diff.max() <= MAX_DEV_LIMIT
            if len(sel) >= 40:
                assert beyond.mean() <= ROWS_BEYOND_LIMIT["e4m3_mfma"]


CASES = [
    # B, H, Hkv, N, d, order, S, delta, n_split
    (1, 1, 1, 1024, 64, "reverse", 256.0, 8.0, 1),
    (1, 1, 1, 1024, 64, "forward", 1.0, 8.0, 4),
    (1, 1, 1, 1024, 64, "reverse", 448.0, 10.0, 16),           # one block per split
    (2, 8, 2, 4096, 128, "reverse", 256.0, 10.0, 8),
    (1, 32, 8, 8192, 128, "forward", 16.0, 12.0, 37),          # uneven split sizes
    (1, 80, 2, 2048, 64, "reverse", 256.0, 8.0, 5),            # 40 query heads per KV head: two groups
    (2, 4, 4, 2048, 256, "reverse", 256.0, 10.0, 6),
    (1, 6, 3, 640, 128, "forward", 3.0, 0.0, 10),              # S not a power of two, no sink
]


@pytest.mark.parametrize("B,H,Hkv,N,d,order,S,delta,n_split", CASES)
def test_decode_parity(B, H, Hkv, N, d, order, S, delta, n_split):
    inp = _decode_inputs(B, H, Hkv, N, d, delta, seed=N + d + n_split)
    t = to_device(inp)
    label = f"decode B{B} H{H} Hkv{Hkv} N{N} d{d} {order} S={S} splits={n_split}"
    say(f"case {label}")
    o = binding.decode(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], kv_order=order, S=S, n_split=n_split)
    torch.cuda.synchronize()
    _check(inp, o, order=order, S=S, n_split=n_split, label=label)



def _random_cases(n=10, seed=31):
    """Seeded random decode shapes: query groups from 1 to 40 heads per KV head, split
    counts from 1 to every block, both orders, S powers of two and not.
    FP8ATTN_DECODE_CASES and FP8ATTN_DECODE_SEED widen or reseed them (default 10, 31)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.integers(1, 4))
        H = Hkv * int(rng.choice([1, 4, 8, 40]))
        N = 64 * int(rng.integers(1, 33 if d < 256 else 17))
        order = str(rng.choice(["forward", "reverse"]))
        S = float(rng.choice([1.0, 256.0, 7.0, 448.0]))
        delta = float(rng.choice([0.0, 8.0, 12.0]))
        n_split = int(rng.integers(1, N // 64 + 1))
        out.append((1, H, Hkv, N, d, order, S, delta, n_split))
    return out


@pytest.mark.parametrize("B,H,Hkv,N,d,order,S,delta,n_split",
                         _random_cases(n=int(os.environ.get("FP8ATTN_DECODE_CASES", "10")),
                                       seed=int(os.environ.get("FP8ATTN_DECODE_SEED", "31"))))
def test_decode_random_parity(B, H, Hkv, N, d, order, S, delta, n_split):
    test_decode_parity(B, H, Hkv, N, d, order, S, delta, n_split)

def test_decode_long_context_default_splits():
    """The measured decode workload's shape (B=1, 32 query heads over 8 KV heads,
    N = 131072, d = 128) with the default split count; four heads checked in full (the
    first and last of the first KV head, one in the middle, the last head)."""
    w = I.WORKLOADS["decode_gqa_h32_kv8_n131072_d128"]
    inp = I.make_workload_inputs(w, seed=0, keep_float=False)
    t = to_device(inp)
    n_split = binding.decode_default_splits(w.B, w.Hkv, w.H, w.N)
    label = f"{w.name} splits={n_split}"
    say(f"case {label}")
    o = binding.decode(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], kv_order="reverse", S=256.0)
    torch.cuda.synchronize()
    _check(inp, o, order="reverse", S=256.0, n_split=n_split, label=label,
           heads=[(0, 0), (0, 3), (0, 17), (0, 31)])


def test_decode_deterministic_and_workspace_reuse():
    inp = _decode_inputs(1, 8, 2, 4096, 128, 10.0, seed=3)
    t = to_device(inp)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=t["q8"].device)
    say("case decode determinism")
    a = binding.decode(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], n_split=16, workspace=ws)
    b = binding.decode(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], n_split=16, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decode_static_default_splits_fit_the_scratch():
    """Without n_split, decode_static lowers the default split count to what the static
    scratch holds: one KV head of N = 262144 keys with 32 query heads gets 512 splits by
    default (8.6 MB of records), and the 8 MiB scratch holds 496. The result is bitwise equal
    to the workspace decode at 496 splits."""
    B, H, Hkv, N, d = 1, 32, 1, 262144, 128
    assert binding.decode_default_splits(B, Hkv, H, N) == 512
    fit = binding.STATIC_SCRATCH_BYTES // binding.load().fp8_attn_decode_workspace_bytes(B, H, d, 1)
    assert fit == 496
    inp = _decode_inputs(B, H, Hkv, N, d, 10.0, seed=77)
    t = to_device(inp)
    say(f"case static-scratch decode B{B} H{H} Hkv{Hkv} N{N} d{d}, default splits")
    args = (t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"])
    got = binding.decode_static(*args, kv_order="reverse", S=256.0)
    ref = binding.decode(*args, kv_order="reverse", S=256.0, n_split=fit)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
