"""The three shapes of the forward kernel at d = 128 (GPU), each against the oracle.

With C compute units and T = B H ceil(N / 128) tiles of 128 query rows, the library picks:
- two walk groups (``fp8_attn_fwd_walk_groups`` = 2): 64-row tiles of 4 waves, two groups
  of 2 waves splitting the KV walk and trading block row maxima through LDS, when
  2 T <= 3 C with causal masking or 2 T <= C without;
- 16 query rows per wave (``fp8_attn_fwd_tile_rows`` = 16; fwd16.hip: Q.K^T on
  v_mfma_f32_16x16x128_f8f6f4, P.V on v_mfma_f32_16x16x32_fp8_fp8, 64-row workgroups) when
  1.5 C < T <= 2 C with causal masking;
- otherwise 32 rows per wave, one group (fwd.hip).

Every case first asserts which shape the library picks, then checks the output and the
counts against the exact-logit oracle (and the device-logit one) with the tolerance of the
other parity tests: the walk groups produce the P~ of the sequential walk (only the fp32
summation order of O changes), and the same logit-error bound holds for both Q.K^T
instructions (``tests/test_gpu_hw_probe.py``). The small d = 128 cases of the other parity
files run on the walk groups too.
"""
import numpy as np
import pytest
import torch

from precision_attention_amd import binding
from precision_attention_amd import inputs as I

from _gpu_util import check_both, check_counts, oracle, pair_counts, say, to_device

pytestmark = pytest.mark.gpu


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _tiles(B, H, N):
    return B * H * ((N + 127) // 128)


def expected_groups(B, H, N, causal, cus):
    t = _tiles(B, H, N)
    return 2 if (2 * t <= 3 * cus if causal else 2 * t <= cus) else 1


def expected_rows(B, H, N, causal, cus):
    if expected_groups(B, H, N, causal, cus) == 2:
        return 32
    return 16 if causal and _tiles(B, H, N) <= 2 * cus else 32


def test_routing():
    cus = _cus()
    for B, H, N in ((1, 8, 4096), (1, 2, 4096), (1, 4, 8192), (1, 16, 8192), (2, 4, 4096), (1, 32, 32768),
                    (1, 7, 8192), (4, 26, 512)):
        for causal in (False, True):
            assert binding.fwd_walk_groups(B, H, H, N, 128, causal=causal) == expected_groups(B, H, N, causal, cus)
            assert binding.fwd_tile_rows(B, H, H, N, 128, causal=causal) == expected_rows(B, H, N, causal, cus)
    small = dict(B=1, H=2, Hkv=2, N=4096, d=128)
    assert binding.fwd_walk_groups(**small) == expected_groups(1, 2, 4096, True, cus)
    for kw in (dict(kv_order="reverse_sink_last"), dict(denominator="quantized"), dict(exact_qk=True)):
        assert binding.fwd_walk_groups(**small, **kw) == 1
        assert binding.fwd_tile_rows(**small, **kw) == 32
    for d in (64, 256):
        assert binding.fwd_walk_groups(1, 2, 2, 4096, d) == 1
        assert binding.fwd_tile_rows(1, 8, 8, 4096, d) == 32
    if cus == 256:
        # the thresholds on MI355X: walk groups up to 384 tiles with causal masking and up to
        # 128 without, 16-row waves from 385 to 512 causal tiles
        assert binding.fwd_walk_groups(1, 12, 4, 4096, 128, causal=True) == 2        # 384 tiles
        assert binding.fwd_walk_groups(1, 12, 4, 4160, 128, causal=True) == 1        # 396
        assert binding.fwd_tile_rows(1, 12, 4, 4160, 128, causal=True) == 16         # 396
        assert binding.fwd_tile_rows(1, 16, 4, 4096, 128, causal=True) == 16         # 512
        assert binding.fwd_tile_rows(1, 16, 4, 4160, 128, causal=True) == 32         # 528
        assert binding.fwd_walk_groups(1, 4, 4, 4096, 128, causal=False) == 2        # 128
        assert binding.fwd_walk_groups(1, 4, 4, 4160, 128, causal=False) == 1       # 132
        assert binding.fwd_tile_rows(1, 4, 4, 4160, 128, causal=False) == 32         # 132
        assert binding.fwd_walk_groups(1, 8, 8, 4096, 128, causal=False) == 1        # the sweep shape
        assert binding.fwd_tile_rows(1, 8, 8, 4096, 128, causal=False) == 32


def _run(B, H, Hkv, N, causal, order, S, delta, *, rows_expected, groups_expected=1, sample_rows=None,
         heads=None, seed=0):
    d = 128
    assert binding.fwd_tile_rows(B, H, Hkv, N, d, causal=causal, kv_order=order, S=S) == rows_expected
    assert binding.fwd_walk_groups(B, H, Hkv, N, d, causal=causal, kv_order=order, S=S) == groups_expected
    inp = I.make_inputs(B, H, Hkv, N, d, delta=delta, seed=seed, descale="head",
                        keep_float=False)
    t = to_device(inp)
    label = (f"B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} {order} S={S} delta={delta} "
             f"({rows_expected}-row waves, {groups_expected} walk group(s))")
    say(f"case {label}")
    o, c = binding.fwd_counted(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=causal,
                               kv_order=order, S=S, n_sink=4)
    c_only = binding.p_collapse_count(t["q8"], t["k8"], t["qd"], t["kd"], causal=causal, kv_order=order,
                                      S=S, n_sink=4)
    o_plain = binding.fwd(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=causal, kv_order=order,
                          S=S)
    torch.cuda.synchronize()
    c = c.cpu().numpy().astype(np.int64)
    assert np.array_equal(c, c_only.cpu().numpy().astype(np.int64)), "fused and count-only counts differ"
    assert torch.equal(o, o_plain), "fused and plain forward differ"
    assert tuple(c[2:]) == pair_counts(B, H, N, causal)
    rows = None if sample_rows is None else I.sample_rows(N, sample_rows, seed=seed)
    check_both(inp, o, c if sample_rows is None else None, causal=causal, order=order, S=S, label=label,
               rows=rows, heads=heads)
    return inp, t


PAIRS = [
    # B, H, Hkv, N, causal, order, S, delta: small grids, two walk groups
    (1, 1, 1, 64, False, "forward", 256.0, 8.0),           # one block: group 1 has nothing to walk
    (1, 1, 1, 64, True, "reverse", 256.0, 8.0),
    (1, 1, 1, 128, True, "reverse", 256.0, 8.0),           # two blocks, one per group
    (1, 2, 1, 192, True, "reverse", 448.0, 10.0),          # odd block count, GQA
    (1, 2, 2, 192, False, "forward", 1.0, 6.0),
    (2, 2, 1, 320, True, "forward", 3.0, 7.0),             # S not a power of two
    (1, 8, 2, 256, True, "forward", 1.0, 0.0),             # no sink at all
    (1, 4, 4, 1024, False, "reverse", 16.0, 12.0),
    (3, 2, 1, 640, True, "reverse", 256.0, 10.0),
    (1, 2, 2, 2048, True, "reverse", 100.0, 8.0),          # S on an E4M3 midpoint
]


@pytest.mark.parametrize("B,H,Hkv,N,causal,order,S,delta", PAIRS)
def test_walk_groups_full_parity(B, H, Hkv, N, causal, order, S, delta):
    if expected_groups(B, H, N, causal, _cus()) != 2:
        pytest.skip("this device runs the shape on one walk group")
    _run(B, H, Hkv, N, causal, order, S, delta, rows_expected=32, groups_expected=2, seed=B * 100 + N)


ROWS16 = [
    # causal grids of 385 to 512 tiles of 128 rows on MI355X: 16-row waves (many short heads)
    (4, 100, 25, 128, True, "reverse", 256.0, 10.0),       # 400 tiles
    (2, 104, 26, 192, True, "forward", 3.0, 7.0),          # 416 tiles, ragged last tile
    (1, 200, 50, 256, True, "reverse", 448.0, 8.0),        # 400 tiles
]


@pytest.mark.parametrize("B,H,Hkv,N,causal,order,S,delta", ROWS16)
def test_rows16_full_parity(B, H, Hkv, N, causal, order, S, delta):
    if expected_rows(B, H, N, causal, _cus()) != 16:
        pytest.skip("this device runs the shape on another kernel shape")
    _run(B, H, Hkv, N, causal, order, S, delta, rows_expected=16, seed=B * 100 + N)


def test_medium_grids_sampled():
    """Non-causal H4 N4096 (128 tiles: two walk groups; sampled rows of two heads, counts of
    all heads against the oracle) and causal H8 N8192 (512 tiles: 16-row waves; sampled
    rows)."""
    cus = _cus()
    if expected_groups(1, 4, 4096, False, cus) == 2:
        inp, t = _run(1, 4, 4, 4096, False, "forward", 256.0, 8.0, rows_expected=32, groups_expected=2,
                      sample_rows=192, heads=[(0, 0), (0, 3)])
        c = binding.p_collapse_count(t["q8"], t["k8"], t["qd"], t["kd"], causal=False, kv_order="forward",
                                     S=256.0, n_sink=4)
        torch.cuda.synchronize()
        ref = oracle(inp, causal=False, order="forward", S=256.0, counts=True)
        check_counts(c.cpu().numpy().astype(np.int64), ref["counts"], ref["zero_flagged"], "H4 N4096 counts")
    if expected_rows(1, 8, 8192, True, cus) == 16:
        _run(1, 8, 8, 8192, True, "reverse", 256.0, 10.0, rows_expected=16, sample_rows=160,
             heads=[(0, 0), (0, 7)], seed=3)


ROWS32 = [
    # grids past the thresholds: the 32-row kernel at d = 128
    (1, 32, 8, 4096, True, "reverse", 256.0, 10.0),
    (1, 16, 16, 4096, False, "forward", 3.0, 7.0),
    (2, 16, 4, 4096, True, "forward", 448.0, 8.0),
]


@pytest.mark.parametrize("B,H,Hkv,N,causal,order,S,delta", ROWS32)
def test_rows32_d128_sampled(B, H, Hkv, N, causal, order, S, delta):
    if expected_rows(B, H, N, causal, _cus()) != 32 or expected_groups(B, H, N, causal, _cus()) != 1:
        pytest.skip("this device runs the shape on another kernel shape")
    _run(B, H, Hkv, N, causal, order, S, delta, rows_expected=32, sample_rows=160,
         heads=[(0, 0), (B - 1, H - 1)], seed=7 + N + H)
