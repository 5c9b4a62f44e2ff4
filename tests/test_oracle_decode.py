"""Pins of the split-KV decode oracle (CPU only): the key ranges, the single-split case
against the prefill recurrence, no cast against the textbook softmax for any split, one
block per split against a brute force written from the closed form (with torch's own E4M3
cast), and the isolation of the sink that splitting brings."""
import math

import numpy as np
import pytest
import torch
from scipy.special import softmax

from oracle import attention as A


def _logits(N, seed, sink=None, scale=2.0):
    s = np.random.default_rng(seed).standard_normal((1, N)) * scale
    if sink is not None:
        s[:, :4] += sink
    return s


def _torch_e4m3(x):
    t = torch.tensor(np.minimum(np.asarray(x, dtype=np.float32), 448.0))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("N,n_split", [(64, 1), (640, 3), (640, 10), (4096, 7), (4096, 64)])
def test_split_ranges_partition_the_blocks(N, n_split):
    r = A.split_ranges(N, n_split)
    assert r[0][0] == 0 and r[-1][1] == N
    assert all(a[1] == b[0] for a, b in zip(r, r[1:]))
    sizes = [(e - s) // 64 for s, e in r]
    assert min(sizes) >= 1 and max(sizes) - min(sizes) <= 1


def test_split_count_bounds():
    with pytest.raises(ValueError):
        A.split_ranges(640, 11)
    with pytest.raises(ValueError):
        A.split_ranges(640, 0)


@pytest.mark.parametrize("order", ["forward", "reverse"])
@pytest.mark.parametrize("S", [1.0, 256.0, 448.0])
def test_one_split_is_the_prefill_recurrence(order, S):
    s = _logits(1024, 1, sink=8.0)
    v = np.random.default_rng(2).standard_normal((1024, 8))
    o_dec = A.decode_split(s, v, kv_order=order, S=S, n_split=1)
    o_pre, _ = A.online_softmax_pcast(s, v, kv_order=order, S=S)
    assert np.abs(o_dec - o_pre).max() < 1e-14


@pytest.mark.parametrize("n_split", [1, 2, 5, 16])
def test_without_cast_any_split_is_the_textbook_softmax(n_split):
    s = _logits(1024, 3, sink=9.0)
    v = np.random.default_rng(4).standard_normal((1024, 8))
    o = A.decode_split(s, v, kv_order="reverse", S=256.0, n_split=n_split, p_cast="none")
    assert np.abs(o - softmax(s, axis=1) @ v).max() < 1e-12


@pytest.mark.parametrize("S", [1.0, 256.0])
def test_one_block_per_split_brute_force(S):
    """Every split holds one block b: its max is the block max m_b, so
    O = sum_b sum_j E4M3(e^(s_j - m_b) S) e^(m_b - m) v_j / (S sum_j e^(s_j - m))."""
    N = 384
    s = _logits(N, 5, sink=7.0)
    v = np.random.default_rng(6).standard_normal((N, 4))
    o = A.decode_split(s, v, kv_order="forward", S=S, n_split=N // 64)[0]
    m = s.max()
    num = np.zeros(4)
    den = 0.0
    for b in range(N // 64):
        mb = s[0, 64 * b:64 * b + 64].max()
        for j in range(64 * b, 64 * b + 64):
            num += float(_torch_e4m3([math.exp(s[0, j] - mb) * S])[0]) * math.exp(mb - m) * v[j]
            den += S * math.exp(s[0, j] - m)
    assert np.abs(o - num / den).max() < 1e-12
    # one block per split: the walk order inside a split cannot matter
    o_rev = A.decode_split(s, v, kv_order="reverse", S=S, n_split=N // 64)[0]
    assert np.array_equal(o, o_rev)


def test_splitting_isolates_the_sink():
    """Forward order, S = 256, sink strength 12: unsplit, every non-sink P is cast under
    the sink's max and a fraction of them collapses; split, only the first split's keys
    ever see that max, so every collapse lies in the first split."""
    N = 4096
    s = _logits(N, 7, sink=12.0, scale=1.0)
    zeros_unsplit = A.collapse_counts(s, kv_order="forward", S=256.0, n_sink=4)[0]
    per_split = []
    for k, (j0, j1) in enumerate(A.split_ranges(N, 64)):
        per_split.append(A.collapse_counts(s[:, j0:j1], kv_order="forward", S=256.0, n_sink=4 if k == 0 else 0)[0])
    assert zeros_unsplit > 1000
    assert sum(per_split[1:]) == 0
    assert per_split[0] <= 60
