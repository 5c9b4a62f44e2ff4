"""The library's launches captured in a HIP graph (torch.cuda.CUDAGraph on the capture
stream) and replayed: every replay must give, bit for bit, what the same call gives
eagerly. Between replays the test runs other eager work, overwrites the outputs, the
collapse counters and the workspaces with garbage, and loads new inputs into the captured
input buffers, so a replay that reused stale memory, skipped the in-graph counter reset or
read the inputs of the capture would show. The entry points enqueue kernels only (no
memset nodes, no allocation, no host synchronisation), which is what makes them
capturable; the static-scratch decode is the one meant for callers that cannot allocate."""
import numpy as np
import pytest
import torch

from precision_attention_amd import binding
from precision_attention_amd import inputs as I

from _gpu_util import say, to_device

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _fill_inputs(dst, B, H, Hkv, N, d, seed, *, decode=False):
    """New seeded inputs written into the existing device tensors of ``dst``."""
    inp = I.make_inputs(B, H, Hkv, N, d, delta=8.0, seed=seed, descale="head", keep_float=False,
                        n_q=1 if decode else None)
    if decode:
        inp["q8"] = np.ascontiguousarray(inp["q8"][:, :, 0, :])
    src = to_device(inp)
    for k in ("q8", "k8", "v8", "qd", "kd", "vd"):
        dst[k].copy_(src[k])


def _new_inputs(B, H, Hkv, N, d, seed, *, decode=False):
    inp = I.make_inputs(B, H, Hkv, N, d, delta=8.0, seed=seed, descale="head", keep_float=False,
                        n_q=1 if decode else None)
    if decode:
        inp["q8"] = np.ascontiguousarray(inp["q8"][:, :, 0, :])
    return to_device(inp)


def _capture(fn):
    """Warm up on a side stream, then capture one call of ``fn`` (which launches on the
    current stream) into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(name, g, t, shape, seeds, eager, outs, scratch, *, decode=False):
    """For each seed: new inputs into the captured buffers, eager reference into separate
    buffers, garbage into the captured outputs and scratch, other eager work, one replay,
    and a bitwise comparison of every output."""
    B, H, Hkv, N, d = shape
    other = _new_inputs(1, 2, 1, 256, 64, seed=7)
    for rep, seed in enumerate(seeds):
        _fill_inputs(t, B, H, Hkv, N, d, seed, decode=decode)
        ref = [x.clone() for x in eager()]
        for x in outs:
            if x.dtype.is_floating_point:
                x.fill_(float("nan"))
            else:
                x.fill_(123456789)
        for x in scratch:
            x.fill_(0xA5)
        binding.fwd(other["q8"], other["k8"], other["v8"], other["qd"], other["kd"], other["vd"],
                    causal=False, kv_order="forward", S=16.0)       # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            same = torch.equal(got, want)
            say(f"  {name} replay {rep} (inputs seed {seed}) output {i}: {'bitwise equal' if same else 'DIFFERS'}")
            assert same, f"{name}: replay {rep} output {i} differs from the eager call"


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [(1, 4, 2, 1024, 128, True), (2, 2, 2, 512, 64, False)])
def test_fwd_counted_replays_equal_eager(B, H, Hkv, N, d, causal):
    say(f"case graph capture: fwd_counted B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    t = _new_inputs(B, H, Hkv, N, d, seed=1)
    dev = t["q8"].device
    o = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    c = torch.empty(4, dtype=torch.int64, device=dev)
    args = lambda: (t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"])   # noqa: E731
    call = lambda out, counts: binding.fwd_counted(*args(), causal=causal, kv_order="reverse", S=256.0,  # noqa: E731
                                                   n_sink=4, out=out, counts=counts)
    eager = lambda: call(torch.empty_like(o), torch.empty_like(c))   # noqa: E731
    g = _capture(lambda: call(o, c))
    _replay_and_check("fwd_counted", g, t, (B, H, Hkv, N, d), range(11, 11 + REPLAYS), eager, [o, c], [])


def test_fwd_exact_qk_replays_equal_eager():
    B, H, Hkv, N, d = 1, 4, 1, 512, 128
    say(f"case graph capture: fwd_exact_qk (key conversion + count reset + forward) B{B} H{H} Hkv{Hkv} N{N} d{d}")
    t = _new_inputs(B, H, Hkv, N, d, seed=2)
    dev = t["q8"].device
    lib = binding.load()
    o = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    c = torch.empty(4, dtype=torch.int64, device=dev)
    ws = torch.empty(int(lib.fp8_attn_fwd_exact_qk_workspace_bytes(B, Hkv, N, d)), dtype=torch.uint8, device=dev)

    def call(out, counts, workspace):
        return binding.fwd_exact_qk(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=True,
                                    kv_order="reverse", S=256.0, n_sink=4, count=True, out=out, counts=counts,
                                    workspace=workspace)

    eager = lambda: call(torch.empty_like(o), torch.empty_like(c), torch.empty_like(ws))   # noqa: E731
    g = _capture(lambda: call(o, c, ws))
    _replay_and_check("fwd_exact_qk", g, t, (B, H, Hkv, N, d), range(21, 21 + REPLAYS), eager, [o, c], [ws])


@pytest.mark.parametrize("static", [False, True])
def test_decode_replays_equal_eager(static):
    B, H, Hkv, N, d, n_split = 2, 8, 2, 4096, 128, 8
    name = "decode_static" if static else "decode"
    say(f"case graph capture: {name} (split pass + merge) B{B} H{H} Hkv{Hkv} N{N} d{d} splits={n_split}")
    t = _new_inputs(B, H, Hkv, N, d, seed=3, decode=True)
    dev = t["q8"].device
    lib = binding.load()
    o = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    ws = torch.empty(int(lib.fp8_attn_decode_workspace_bytes(B, H, d, n_split)), dtype=torch.uint8, device=dev)
    args = lambda: (t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"])   # noqa: E731
    if static:
        call = lambda out: (binding.decode_static(*args(), kv_order="reverse", S=256.0, n_split=n_split,  # noqa: E731
                                                  out=out),)
        scratch = []
    else:
        call = lambda out, workspace=ws: (binding.decode(*args(), kv_order="reverse", S=256.0,  # noqa: E731
                                                         n_split=n_split, out=out, workspace=workspace),)
        scratch = [ws]
    if static:
        eager = lambda: call(torch.empty_like(o))   # noqa: E731
    else:
        eager = lambda: call(torch.empty_like(o), torch.empty_like(ws))   # noqa: E731
    g = _capture(lambda: call(o))
    _replay_and_check(name, g, t, (B, H, Hkv, N, d), range(31, 31 + REPLAYS), eager, [o], scratch, decode=True)
