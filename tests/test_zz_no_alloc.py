"""fp8_attn_decode_static (the decode entry point that allocates nothing: its split records
live in the library's static per-GPU scratch) against fp8_attn_decode with a caller
workspace, through the C ABI: bit for bit on two calls in a row, the second with a smaller
input (the array keeps the first call's records, which the second must not read), and a
request beyond the array refused with FP8ATTN_ESCRATCH before any launch."""
import numpy as np
import pytest
import torch

from precision_attention_amd import binding
from precision_attention_amd import inputs as I

from _gpu_util import say, to_device

pytestmark = pytest.mark.gpu

FP8ATTN_ESCRATCH = -4
STATIC_SCRATCH_BYTES = 8 << 20


def _inputs(B, H, Hkv, N, d, delta, seed):
    inp = I.make_inputs(B, H, Hkv, N, d, delta=delta, seed=seed, descale="head", keep_float=False, n_q=1)
    inp["q8"] = np.ascontiguousarray(inp["q8"][:, :, 0, :])
    return to_device(inp)


def test_static_scratch_decode_matches_workspace_decode():
    cases = [
        # B, H, Hkv, N, d, order, S, delta, n_split: the second smaller in every size
        (2, 32, 8, 8192, 128, "reverse", 256.0, 10.0, 32),
        (1, 8, 2, 2048, 64, "forward", 16.0, 8.0, 5),
    ]
    for (B, H, Hkv, N, d, order, S, delta, n_split) in cases:
        need = binding.load().fp8_attn_decode_workspace_bytes(B, H, d, n_split)
        assert need <= STATIC_SCRATCH_BYTES
        say(f"case static-scratch decode B{B} H{H} Hkv{Hkv} N{N} d{d} {order} S={S} splits={n_split} ({need} B)")
        t = _inputs(B, H, Hkv, N, d, delta, seed=N + d)
        args = (t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"])
        ref = binding.decode(*args, kv_order=order, S=S, n_split=n_split)
        got = binding.decode_static(*args, kv_order=order, S=S, n_split=n_split)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref), float((got - ref).abs().max())


def test_static_scratch_request_beyond_the_array_is_refused():
    lib = binding.load()
    B, H, d, n_split = 8, 64, 256, 64
    assert lib.fp8_attn_decode_workspace_bytes(B, H, d, n_split) > STATIC_SCRATCH_BYTES
    say("case static-scratch decode: oversize request")
    t = _inputs(1, 1, 1, 64, 64, 8.0, seed=1)        # valid pointers; nothing may be launched
    o = torch.empty(16, dtype=torch.float32, device=t["q8"].device)
    rc = lib.fp8_attn_decode_static(t["q8"].data_ptr(), t["k8"].data_ptr(), t["v8"].data_ptr(), o.data_ptr(),
                                    B, H, H, 64 * n_split, d, 1, 256.0, t["qd"].data_ptr(), t["kd"].data_ptr(),
                                    t["vd"].data_ptr(), n_split, None)
    assert rc == FP8ATTN_ESCRATCH
    assert lib.fp8_attn_status_string(rc).startswith(b"request exceeds")
