"""Pins of the oracle's two schedule/denominator options (CPU only).

* "reverse_sink_last": the reverse walk with block 0 visited as its non-sink keys
  [n_sink, 64) and then the sink keys [0, n_sink). Pinned by: the unit list covering
  every key exactly once, n_sink = 0 reducing to plain reverse, the textbook softmax
  when nothing is cast, a pure-Python brute force, and the property the schedule exists
  for (no non-sink P cast after the sink raised the running max, so clean inputs show
  no collapse at all).
* denominator "quantized": l sums the decoded cast operand. Pinned by: the textbook
  softmax when nothing is cast, O being an exact convex combination of V with the
  decoded codes as weights (brute force with torch's own E4M3 cast), and the
  recurrence agreeing with its closed form.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import softmax

from oracle import attention as A
from precision_attention_amd import inputs as I


def _rand_logits(R, N, seed, scale=2.0, causal=False, sink=None, n_sink=4):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((R, N)) * scale
    if sink is not None:
        s[:, :n_sink] += sink
    if causal:
        s = np.where(np.arange(N)[None, :] > np.arange(R)[:, None], -np.inf, s)
    return s


def _torch_e4m3(x):
    """Round to E4M3FN with torch's CPU cast (saturating at 448 first): a rounding path
    that shares nothing with the oracle's codec."""
    t = torch.tensor(np.minimum(np.asarray(x, dtype=np.float32), 448.0))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


# ------------------------------------------------------------------ visit units

@pytest.mark.parametrize("order", ["forward", "reverse", "reverse_sink_last"])
@pytest.mark.parametrize("n_sink", [0, 1, 4, 63, 64])
def test_units_cover_every_key_once(order, n_sink):
    N = 256
    units = A.visit_units(N, order, n_sink=n_sink)
    seen = np.zeros(N, dtype=int)
    for j0, j1 in units:
        assert 0 <= j0 < j1 <= N
        seen[j0:j1] += 1
    assert (seen == 1).all()
    if order == "reverse_sink_last":
        tail = [u for u in ((n_sink, 64), (0, n_sink)) if u[1] > u[0]]
        assert units[-len(tail):] == tail
        assert units[:-len(tail)] == [(64 * b, 64 * b + 64) for b in range(N // 64 - 1, 0, -1)]


def test_sink_last_rejects_sinks_beyond_a_block():
    with pytest.raises(ValueError):
        A.visit_units(256, "reverse_sink_last", n_sink=65)


def test_sink_last_with_no_sinks_is_reverse():
    s = _rand_logits(64, 256, 1, causal=True, sink=8.0)
    v = np.random.default_rng(2).standard_normal((256, 8))
    a, _ = A.online_softmax_pcast(s, v, kv_order="reverse", S=256.0)
    b, _ = A.online_softmax_pcast(s, v, kv_order="reverse_sink_last", S=256.0, n_sink=0)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("order", ["forward", "reverse", "reverse_sink_last"])
@pytest.mark.parametrize("denominator", ["fp32", "quantized"])
@pytest.mark.parametrize("causal", [False, True])
def test_without_cast_every_variant_is_the_textbook_softmax(order, denominator, causal):
    s = _rand_logits(128, 192, 3, causal=causal, sink=7.0)
    v = np.random.default_rng(4).standard_normal((192, 8))
    o, _ = A.online_softmax_pcast(s, v, kv_order=order, S=256.0, p_cast="none", denominator=denominator)
    assert np.abs(o - softmax(s, axis=1) @ v).max() < 1e-12


# ------------------------------------------------------------------ brute force

def _brute_row(s_row, v, units, S, denominator):
    """Pure-Python recurrence over the given key ranges, E4M3 by torch's cast."""
    d = v.shape[1]
    m, l, acc = -math.inf, 0.0, [0.0] * d
    for j0, j1 in units:
        keys = [j for j in range(j0, j1) if s_row[j] != -math.inf]
        if not keys:
            continue
        m_new = max(m, max(s_row[j] for j in keys))
        alpha = 0.0 if m == -math.inf else math.exp(m - m_new)
        l *= alpha
        acc = [a * alpha for a in acc]
        for j in keys:
            p = math.exp(s_row[j] - m_new)
            p8 = float(_torch_e4m3([p * S])[0])
            l += p * S if denominator == "fp32" else p8
            for c in range(d):
                acc[c] += p8 * v[j, c]
        m = m_new
    return [a / l for a in acc]


@pytest.mark.parametrize("order,S,causal,denominator", [
    ("reverse_sink_last", 256.0, True, "fp32"), ("reverse_sink_last", 1.0, False, "quantized"),
    ("forward", 448.0, True, "quantized"), ("reverse", 16.0, False, "quantized")])
def test_brute_force_python_loops(order, S, causal, denominator):
    s = _rand_logits(20, 128, 8, scale=2.5, causal=causal, sink=6.0)
    v = np.random.default_rng(9).standard_normal((128, 4))
    n_sink = 4
    o, _ = A.online_softmax_pcast(s, v, kv_order=order, S=S, n_sink=n_sink, denominator=denominator)
    # units written out independently of visit_units
    if order == "forward":
        units = [(0, 64), (64, 128)]
    elif order == "reverse":
        units = [(64, 128), (0, 64)]
    else:
        units = [(64, 128), (n_sink, 64), (0, n_sink)]
    for i in range(s.shape[0]):
        assert np.abs(o[i] - _brute_row(s[i], v, units, S, denominator)).max() < 1e-12


@pytest.mark.parametrize("order", ["forward", "reverse", "reverse_sink_last"])
@pytest.mark.parametrize("denominator", ["fp32", "quantized"])
@pytest.mark.parametrize("causal", [False, True])
def test_sequential_equals_closed_form(order, denominator, causal):
    s = _rand_logits(192, 384, 11, scale=1.5, causal=causal, sink=9.0)
    v = np.random.default_rng(12).standard_normal((384, 8))
    o, _ = A.online_softmax_pcast(s, v, kv_order=order, S=256.0, denominator=denominator)
    ov = A.online_softmax_pcast_vectorized(s, v, kv_order=order, S=256.0, denominator=denominator)
    assert np.abs(o - ov).max() < 1e-12


def test_quantized_denominator_is_a_convex_combination():
    """With one block, O = sum_j dec(P8_j) v_j / sum_j dec(P8_j): the weights are exactly the
    decoded codes, so a V that is constant per column is returned unchanged, and a one-hot
    V column returns that key's normalised code."""
    s = _rand_logits(8, 64, 21, scale=3.0)
    S = 256.0
    p = np.exp(s - s.max(axis=1, keepdims=True))
    codes = _torch_e4m3(p * S)
    w = codes / codes.sum(axis=1, keepdims=True)
    v = np.zeros((64, 3))
    v[:, 0] = 2.5            # constant column
    v[17, 1] = 1.0           # one-hot column
    v[:, 2] = np.arange(64)  # ramp
    o, _ = A.online_softmax_pcast(s, v, kv_order="forward", S=S, denominator="quantized")
    assert np.abs(o[:, 0] - 2.5).max() < 1e-14
    assert np.abs(o[:, 1] - w[:, 17]).max() < 1e-15
    assert np.abs(o[:, 2] - w @ np.arange(64)).max() < 1e-12


# ------------------------------------------------------------------ what the schedule is for

@pytest.mark.parametrize("delta", [8.0, 10.0, 12.0])
def test_sink_last_removes_the_sink_block_collapse(delta):
    """Clean sinks (N = 1024, d = 64, S = 256): plain reverse still casts the 60 non-sink
    keys of block 0 under the sink's max and collapses some of them; visiting them before
    the sinks leaves no non-sink P cast under a sink max, and none collapses."""
    inp = I.make_inputs(1, 1, 1, 1024, 64, delta=delta, seed=0, descale="tensor", keep_float=False)
    s, _ = A.head_logits_e4m3(inp["q8"][0, 0], inp["k8"][0, 0], inp["qd"][0, 0], inp["kd"][0, 0], 64)
    rev = A.collapse_counts(s, kv_order="reverse", S=256.0, n_sink=4)
    last = A.collapse_counts(s, kv_order="reverse_sink_last", S=256.0, n_sink=4)
    assert rev[1] > 0 and rev[0] == rev[1]
    assert last[0] == 0
    assert last[2] == rev[2] and last[3] == rev[3]      # same pairs, only the order differs
