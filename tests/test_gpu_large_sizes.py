"""GPU parity at sizes whose tensors hold more than 2^31 elements, where element offsets
overflow 32-bit arithmetic: a causal GQA prefill with 80 query heads of N = 262144 keys
(Q: 2.7e9 codes, O: 10.7 GB) and a split-KV decode over 80 KV heads of N = 262144 keys
(K and V: 2.7e9 codes each). The first head and the last (the largest offsets) are checked
against the exact-logit oracle on sampled rows (prefill) or in full (decode); the counts
against the closed-form pair totals.

The inputs are drawn head by head on the GPU from a seeded torch generator (generating
2.7e9 values on the host would take minutes and tens of GB): N(0, 1) values, column 0 of
the first 4 tokens of Q and K set to alpha = sqrt(delta sqrt(d)) (the literal sink
construction), a per-head descale amax / 448 and the RNE cast to E4M3. The oracle receives
the codes and descales of the heads it checks."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from precision_attention_amd import binding

from _gpu_util import MAX_DEV_LIMIT, O_TOL, check_output, oracle, pair_counts, say

pytestmark = pytest.mark.gpu

N_SINK = 4


def _e4m3_heads(g, n_heads, n, d, alpha, dev):
    """Codes [1, n_heads, n, d] (uint8) and descales [1, n_heads], one head at a time."""
    codes = torch.empty((1, n_heads, n, d), dtype=torch.uint8, device=dev)
    desc = torch.empty((1, n_heads), dtype=torch.float32, device=dev)
    for h in range(n_heads):
        x = torch.randn((n, d), generator=g, device=dev)
        if alpha is not None:
            x[:N_SINK, 0] = alpha
        s = x.abs().max() / 448.0
        codes[0, h] = (x / s).to(torch.float8_e4m3fn).view(torch.uint8)
        desc[0, h] = s
    return codes, desc


def _host(t):
    return np.ascontiguousarray(t.cpu().numpy())


def test_prefill_beyond_2_31_elements():
    B, H, Hkv, N, d, S, delta = 1, 80, 8, 262144, 128, 256.0, 10.0
    assert B * H * N * d > 2 ** 31
    dev = torch.device("cuda:0")
    label = f"prefill B{B} H{H} Hkv{Hkv} N{N} d{d} causal reverse S={S}"
    say(f"case {label}: drawing inputs")
    g = torch.Generator(device=dev)
    g.manual_seed(2031)
    alpha = math.sqrt(delta * math.sqrt(d))
    q8, qd = _e4m3_heads(g, H, N, d, alpha, dev)
    k8, kd = _e4m3_heads(g, Hkv, N, d, alpha, dev)
    v8, vd = _e4m3_heads(g, Hkv, N, d, None, dev)
    say(f"case {label}: fused forward + count")
    o, c = binding.fwd_counted(q8, k8, v8, qd, kd, vd, causal=True, kv_order="reverse", S=S, n_sink=N_SINK)
    torch.cuda.synchronize()
    counts = c.cpu().numpy().astype(np.int64)
    tot, sink = pair_counts(B, H, N, True, n_sink=N_SINK)
    say(f"  counts {list(counts)}; pre-sink-block collapse {counts[0] - counts[1]} of {tot - sink} pairs")
    assert (int(counts[2]), int(counts[3])) == (tot, sink)
    assert 0 <= counts[1] <= counts[0]
    rows = np.concatenate([np.arange(32), np.arange(N - 16, N)])
    G = H // Hkv
    for h in (0, H - 1):
        hk = h // G
        sub = {"q8": _host(q8[:, h:h + 1]), "k8": _host(k8[:, hk:hk + 1]), "v8": _host(v8[:, hk:hk + 1]),
               "qd": _host(qd[:, h:h + 1]), "kd": _host(kd[:, hk:hk + 1]), "vd": _host(vd[:, hk:hk + 1])}
        say(f"  head {h} (kv head {hk}): exact-logit oracle on {len(rows)} rows")
        ref = oracle(sub, causal=True, order="reverse", S=S, rows=rows, n_sink=N_SINK)
        worst = check_output(o[:, h:h + 1], ref, f"{label} head {h} [exact logits]")
        assert worst <= MAX_DEV_LIMIT
    del q8, k8, v8, o
    torch.cuda.empty_cache()


def test_decode_beyond_2_31_elements():
    B, H, Hkv, N, d, S, delta = 1, 80, 80, 262144, 128, 256.0, 10.0
    assert B * Hkv * N * d > 2 ** 31
    dev = torch.device("cuda:0")
    n_split = binding.decode_default_splits(B, Hkv, H, N)
    label = f"decode B{B} H{H} Hkv{Hkv} N{N} d{d} reverse S={S} splits={n_split}"
    say(f"case {label}: drawing inputs")
    g = torch.Generator(device=dev)
    g.manual_seed(2032)
    alpha = math.sqrt(delta * math.sqrt(d))
    q8, qd = _e4m3_heads(g, H, 1, d, None, dev)
    k8, kd = _e4m3_heads(g, Hkv, N, d, alpha, dev)
    v8, vd = _e4m3_heads(g, Hkv, N, d, None, dev)
    q8 = q8[:, :, 0, :].contiguous()
    say(f"case {label}: decode")
    o = binding.decode(q8, k8, v8, qd, kd, vd, kv_order="reverse", S=S, n_split=n_split)
    torch.cuda.synchronize()
    for h in (0, H - 1):
        sub = {"q8": _host(q8[:, h:h + 1]), "k8": _host(k8[:, h:h + 1]), "v8": _host(v8[:, h:h + 1]),
               "qd": _host(qd[:, h:h + 1]), "kd": _host(kd[:, h:h + 1]), "vd": _host(vd[:, h:h + 1])}
        ref = A.decode_e4m3(sub["q8"], sub["k8"], sub["v8"], sub["qd"], sub["kd"], sub["vd"], kv_order="reverse",
                            S=S, n_split=n_split, logits="exact", with_allowance=True)
        got = o[0, h].cpu().numpy()
        diff = np.abs(got - ref["o"][0, 0])
        excess = diff - (O_TOL + ref["allow"][0, 0])
        say(f"  {label} head {h} [exact logits]: max|dO| {diff.max():.3g}; worst excess {excess.max():.3g}")
        assert np.isfinite(got).all()
        assert excess.max() <= 0, f"head {h}: exceeds tolerance by {excess.max():.3g}"
        assert diff.max() <= MAX_DEV_LIMIT
    del k8, v8, o
    torch.cuda.empty_cache()
