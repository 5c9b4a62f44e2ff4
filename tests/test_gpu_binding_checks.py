"""The binding refuses caller tensors that would hand the library a bad pointer (a host
tensor, a wrong dtype, a short counter or workspace buffer) with ValueError before any
launch, and the library's output is untouched by such a call."""
import pytest
import torch

from precision_attention_amd import binding
from precision_attention_amd import inputs as I

from _gpu_util import device, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def t():
    return to_device(I.make_inputs(1, 2, 1, 128, 64, delta=8.0, seed=5))


def test_bad_out_tensors_raise_before_launch(t):
    dev = device()
    say("case binding checks: out / counts")
    args = (t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"])
    bad_outs = [torch.empty((1, 2, 128, 64), dtype=torch.float32),                  # host memory
                torch.empty((1, 2, 128, 64), dtype=torch.float16, device=dev),      # dtype
                torch.empty((1, 2, 128, 32), dtype=torch.float32, device=dev),      # shape
                torch.empty((1, 2, 64, 128), dtype=torch.float32, device=dev).transpose(2, 3)]
    for out in bad_outs:
        with pytest.raises(ValueError):
            binding.fwd(*args, causal=True, out=out)
        with pytest.raises(ValueError):
            binding.fwd_counted(*args, causal=True, out=out)
        with pytest.raises(ValueError):
            binding.fwd_ex(*args, causal=True, out=out)
    bad_counts = [torch.zeros(4, dtype=torch.int64),                                  # host memory
                  torch.zeros(4, dtype=torch.int32, device=dev),                      # 32-bit counters
                  torch.zeros(3, dtype=torch.int64, device=dev)]                      # too short
    for c in bad_counts:
        with pytest.raises(ValueError):
            binding.fwd_counted(*args, causal=True, counts=c)
        with pytest.raises(ValueError):
            binding.fwd_ex(*args, causal=True, counts=c)
        with pytest.raises(ValueError):
            binding.p_collapse_count(t["q8"], t["k8"], t["qd"], t["kd"], causal=True, out=c)
    with pytest.raises(ValueError):
        binding.fwd(t["q8"].cpu(), t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=True)
    torch.cuda.synchronize()


def test_bad_decode_buffers_raise_before_launch():
    dev = device()
    say("case binding checks: decode out / workspace")
    inp = I.make_inputs(1, 4, 2, 256, 64, delta=8.0, seed=6, n_q=1)
    inp["q8"] = inp["q8"][:, :, 0, :].copy()
    t = to_device(inp)
    args = (t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"])
    need = binding.load().fp8_attn_decode_workspace_bytes(1, 4, 64, 2)
    with pytest.raises(ValueError):
        binding.decode(*args, n_split=2, workspace=torch.empty(need - 16, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        binding.decode(*args, n_split=2, workspace=torch.empty(need, dtype=torch.uint8))
    with pytest.raises(ValueError):
        binding.decode(*args, n_split=2, out=torch.empty((1, 4, 64), dtype=torch.float32))
    o = binding.decode(*args, n_split=2, workspace=torch.empty(need, dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
