"""GPU parity of the causal 32-row launch in head-major grid order. With one query head per
KV head and a small K/V per head, the workgroups of one head run together on one XCD (so
that head's K/V stays in its L2) and, within the head, longest tile first. These cases cover
both grid mappings (whole KV heads per XCD, and the plain one), odd and even tile counts,
ragged last tiles, a single tile, d = 64, 128 and 256, both block orders, S powers of two
and not, and the three entry points: the forward, the collapse count and the fused pass
(which must agree bitwise with the first two). Each is checked against the exact-logit oracle
and the closed-form pair totals."""
import numpy as np
import pytest
import torch

from precision_attention_amd import binding
from precision_attention_amd import inputs as I

from _gpu_util import (check_both, check_counts, check_output, gpu_counts, gpu_fwd, oracle, pair_counts, say,
                       to_device)

pytestmark = pytest.mark.gpu

CASES = [
    # B, H (= Hkv), N, d, order, S, delta
    (1, 8, 448, 64, "reverse", 256.0, 8.0),     # whole KV heads per XCD; 4 tiles, ragged
    (2, 3, 576, 64, "forward", 16.0, 10.0),     # plain mapping; 5 tiles, ragged
    (1, 8, 384, 256, "reverse", 448.0, 12.0),   # d = 256; 3 tiles
    (1, 1, 128, 256, "forward", 256.0, 8.0),    # a single tile
    (1, 2, 1024, 64, "reverse", 5.0, 6.0),      # S not a power of two; 8 tiles
]


def _run(B, H, N, d, order, S, delta, seed):
    inp = I.make_inputs(B, H, H, N, d, delta=delta, seed=seed, descale="head")
    t = to_device(inp)
    o = gpu_fwd(t, causal=True, order=order, S=S)
    c = gpu_counts(t, causal=True, order=order, S=S)
    o2, c2 = binding.fwd_counted(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=True,
                                 kv_order=order, S=S, n_sink=4)
    torch.cuda.synchronize()
    assert torch.equal(o, o2), "fused pass and forward alone differ"
    assert np.array_equal(c2.cpu().numpy().astype(np.int64), c), "fused pass and count alone differ"
    tot, sink = pair_counts(B, H, N, True)
    assert (int(c[2]), int(c[3])) == (tot, sink)
    return inp, o, c


@pytest.mark.parametrize("B,H,N,d,order,S,delta", CASES)
def test_head_major_causal_full_parity(B, H, N, d, order, S, delta):
    assert binding.fwd_tile_rows(B, H, H, N, d, causal=True, kv_order=order, S=S) == 32
    label = f"head-major B{B} H{H} N{N} d{d} {order} S={S} delta={delta}"
    say(f"case {label}")
    inp, o, c = _run(B, H, N, d, order, S, delta, seed=B * 1000 + N + d)
    check_both(inp, o, c, causal=True, order=order, S=S, label=label)


def test_head_major_d128_grid_past_the_16_row_range():
    """d = 128 takes the 32-row kernel once the grid exceeds two 128-row tiles per compute
    unit: 2 x 88 heads x 3 tiles (odd, ragged) = 528 on 256 compute units, whole KV heads per
    XCD. Exact-logit oracle on every head and row, counts on all heads."""
    B, H, N, d, order, S = 2, 88, 320, 128, "reverse", 256.0
    if binding.fwd_tile_rows(B, H, H, N, d, causal=True, kv_order=order, S=S) != 32:
        pytest.skip("this device has more compute units: the grid runs 16-row waves")
    label = f"head-major B{B} H{H} N{N} d{d} {order} S={S}"
    say(f"case {label}")
    inp, o, c = _run(B, H, N, d, order, S, 10.0, seed=31)
    ref = oracle(inp, causal=True, order=order, S=S, counts=True)
    check_output(o, ref, f"{label} [exact logits]", qk="e4m3_mfma", S=S)
    check_counts(c, ref["counts"], ref["zero_flagged"], f"{label} [exact logits]")
