"""The two shapes of the forward kernel at d = 128 (GPU), each against the oracle.

Small grids run 16 query rows per wave in workgroups of 64 rows (fwd16.hip: Q.K^T on
v_mfma_f32_16x16x128_f8f6f4, P.V on v_mfma_f32_16x16x32_fp8_fp8), the others 32 (fwd.hip):
16 when the 128-row tiles T = B H ceil(N / 128) satisfy T <= 2 C with causal masking or
2 T <= C without (C compute units). Every case first asserts which shape the library picks
(``fp8_attn_fwd_tile_rows``), then checks the output and the counts against the exact-logit
oracle (and the device-logit one) with the tolerance of the other parity tests: the same
error bound holds for both Q.K^T instructions (``tests/test_gpu_hw_probe.py``). The small
d = 128 cases of the other parity files run on the 16-row kernel too; the medium cases here
keep the 32-row kernel at d = 128 under the same checks.
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


def expected_rows(B, H, N, causal, cus):
    tiles = B * H * ((N + 127) // 128)
    return 16 if (tiles <= 2 * cus if causal else 2 * tiles <= cus) else 32


def test_routing():
    cus = _cus()
    for B, H, N in ((1, 8, 4096), (1, 2, 4096), (1, 4, 8192), (1, 16, 8192), (2, 4, 4096), (1, 32, 32768)):
        for causal in (False, True):
            assert binding.fwd_tile_rows(B, H, H, N, 128, causal=causal) == expected_rows(B, H, N, causal, cus)
    small = dict(B=1, H=2, Hkv=2, N=4096, d=128)
    assert binding.fwd_tile_rows(**small) == expected_rows(1, 2, 4096, True, cus)
    assert binding.fwd_tile_rows(1, 8, 8, 4096, 64) == 32
    assert binding.fwd_tile_rows(1, 8, 8, 4096, 256) == 32
    assert binding.fwd_tile_rows(**small, kv_order="reverse_sink_last") == 32
    assert binding.fwd_tile_rows(**small, denominator="quantized") == 32
    assert binding.fwd_tile_rows(**small, exact_qk=True) == 32
    if cus == 256:
        # the thresholds on MI355X: causal up to 512 tiles, not causal up to 128
        assert binding.fwd_tile_rows(1, 16, 4, 4096, 128, causal=True) == 16       # 512 tiles
        assert binding.fwd_tile_rows(1, 16, 4, 4160, 128, causal=True) == 32       # 528
        assert binding.fwd_tile_rows(1, 4, 4, 4096, 128, causal=False) == 16       # 128
        assert binding.fwd_tile_rows(1, 4, 4, 4160, 128, causal=False) == 32       # 132
        assert binding.fwd_tile_rows(1, 8, 8, 4096, 128, causal=False) == 32       # the sweep shape


def _run(B, H, Hkv, N, causal, order, S, delta, *, rows_expected, sample_rows=None, heads=None, seed=0):
    d = 128
    assert binding.fwd_tile_rows(B, H, Hkv, N, d, causal=causal, kv_order=order, S=S) == rows_expected
    inp = I.make_inputs(B, H, Hkv, N, d, delta=delta, seed=seed, descale="head",
                        keep_float=False)
    t = to_device(inp)
    label = f"B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} {order} S={S} delta={delta} ({rows_expected}-row waves)"
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


ROWS16 = [
    # B, H, Hkv, N, causal, order, S, delta
    (1, 1, 1, 64, False, "forward", 256.0, 8.0),
    (1, 1, 1, 64, True, "reverse", 256.0, 8.0),
    (1, 2, 1, 192, True, "reverse", 448.0, 10.0),          # ragged query tile, GQA
    (1, 2, 2, 192, False, "forward", 1.0, 6.0),
    (2, 2, 1, 320, True, "forward", 3.0, 7.0),             # S not a power of two
    (1, 8, 2, 256, True, "forward", 1.0, 0.0),             # no sink at all
    (1, 4, 4, 1024, False, "reverse", 16.0, 12.0),
    (3, 2, 1, 640, True, "reverse", 256.0, 10.0),
    (1, 2, 2, 2048, True, "reverse", 100.0, 8.0),          # S on an E4M3 midpoint
]


@pytest.mark.parametrize("B,H,Hkv,N,causal,order,S,delta", ROWS16)
def test_rows16_full_parity(B, H, Hkv, N, causal, order, S, delta):
    _run(B, H, Hkv, N, causal, order, S, delta, rows_expected=16, seed=B * 100 + N)


def test_rows16_medium_sampled():
    """Non-causal H4 N4096 (128 tiles: sampled rows of two heads, counts of all heads against
    the oracle) and causal H8 N8192 (512 tiles: sampled rows)."""
    if expected_rows(1, 4, 4096, False, _cus()) != 16:
        pytest.skip("this device runs the shape on 32-row waves")
    inp, t = _run(1, 4, 4, 4096, False, "forward", 256.0, 8.0, rows_expected=16, sample_rows=192,
                  heads=[(0, 0), (0, 3)])
    c = binding.p_collapse_count(t["q8"], t["k8"], t["qd"], t["kd"], causal=False, kv_order="forward", S=256.0,
                                 n_sink=4)
    torch.cuda.synchronize()
    ref = oracle(inp, causal=False, order="forward", S=256.0, counts=True)
    check_counts(c.cpu().numpy().astype(np.int64), ref["counts"], ref["zero_flagged"], "H4 N4096 counts")
    if expected_rows(1, 8, 8192, True, _cus()) == 16:
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
    if expected_rows(B, H, N, causal, _cus()) != 32:
        pytest.skip("this device runs the shape on 16-row waves")
    _run(B, H, Hkv, N, causal, order, S, delta, rows_expected=32, sample_rows=160,
         heads=[(0, 0), (B - 1, H - 1)], seed=7 + N + H)
