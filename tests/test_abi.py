"""The C ABI without a GPU: the library loads, exports every function declared in
include/*.h, and validates arguments before any HIP call (so these run on the CPU)."""
import ctypes
import glob
import os
import re

import pytest

from precision_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # a 16-byte aligned non-null address; never dereferenced here


def _declared_functions():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(fp8_attn_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libfp8attn.so is not built; run __graft_entry__.build()")
    return binding.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"fp8_attn_fwd", "fp8_attn_p_collapse_count"} <= set(names)
    raw = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_metadata(lib):
    assert lib.fp8_attn_kv_block() == 64
    assert lib.fp8_attn_version().decode().startswith("fp8attn")
    assert lib.fp8_attn_status_string(0) == b"ok"
    assert lib.fp8_attn_status_string(-2).startswith(b"unsupported")


def _fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, H=2, Hkv=1, N=128, d=128, causal=1, order=1,
         S=256.0, qd=FAKE, kd=FAKE, vd=FAKE):
    return lib.fp8_attn_fwd(q, k, v, o, B, H, Hkv, N, d, causal, order, S, qd, kd, vd, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(qd=None), -1), (dict(kd=None), -1), (dict(vd=None), -1),
    (dict(B=0), -1), (dict(H=-1), -1), (dict(N=0), -1), (dict(d=0), -1),
    (dict(H=3, Hkv=2), -1), (dict(causal=2), -1), (dict(order=2), -1), (dict(order=-1), -1),
    (dict(S=0.0), -1), (dict(S=-1.0), -1), (dict(S=449.0), -1), (dict(S=512.0), -1),
    (dict(S=float("nan")), -1), (dict(S=float("inf")), -1),
    (dict(d=96), -2), (dict(d=32), -2), (dict(N=100), -2), (dict(N=96), -2),
    (dict(q=FAKE + 8), -2), (dict(k=FAKE + 4), -2), (dict(v=FAKE + 1), -2), (dict(o=FAKE + 12), -2),
    (dict(B=1 << 20, H=1 << 10, Hkv=1, N=1 << 14), -2),
])
def test_fwd_validation(lib, kw, status):
    assert _fwd(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(n_sink=-1), -1), (dict(n_sink=129), -1), (dict(counts=None), -1), (dict(q=None), -1),
    (dict(S=500.0), -1), (dict(d=48), -2), (dict(q=FAKE + 2), -2),
])
def test_count_validation(lib, kw, status):
    a = dict(q=FAKE, k=FAKE, B=1, H=2, Hkv=1, N=128, d=128, causal=1, order=1, S=256.0,
             qd=FAKE, kd=FAKE, n_sink=4, counts=FAKE)
    a.update(kw)
    rc = lib.fp8_attn_p_collapse_count(a["q"], a["k"], a["B"], a["H"], a["Hkv"], a["N"], a["d"],
                                       a["causal"], a["order"], a["S"], a["qd"], a["kd"],
                                       a["n_sink"], a["counts"], None)
    assert rc == status


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), -1), (dict(counts=None), -1), (dict(n_sink=-3), -1), (dict(S=0.0), -1),
    (dict(H=5, Hkv=2), -1), (dict(d=80), -2), (dict(N=200), -2), (dict(v=FAKE + 4), -2),
])
def test_fwd_counted_validation(lib, kw, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, H=2, Hkv=1, N=128, d=128, causal=1, order=1, S=256.0,
             qd=FAKE, kd=FAKE, vd=FAKE, n_sink=4, counts=FAKE)
    a.update(kw)
    rc = lib.fp8_attn_fwd_counted(a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["Hkv"], a["N"], a["d"],
                                  a["causal"], a["order"], a["S"], a["qd"], a["kd"], a["vd"], a["n_sink"],
                                  a["counts"], None)
    assert rc == status


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), -1), (dict(v=None), -1), (dict(n_sink=-1), -1), (dict(n_sink=129), -1),
    (dict(order=2, n_sink=65), -1), (dict(order=3), -1), (dict(denominator=2), -1),
    (dict(denominator=-1), -1), (dict(S=0.0), -1), (dict(causal=5), -1),
    (dict(d=80), -2), (dict(N=200), -2), (dict(o=FAKE + 4), -2),
])
def test_fwd_ex_validation(lib, kw, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, H=2, Hkv=1, N=128, d=128, causal=1, order=2, S=256.0,
             qd=FAKE, kd=FAKE, vd=FAKE, n_sink=4, denominator=1, counts=None)
    a.update(kw)
    rc = lib.fp8_attn_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["Hkv"], a["N"], a["d"],
                             a["causal"], a["order"], a["S"], a["qd"], a["kd"], a["vd"], a["n_sink"],
                             a["denominator"], a["counts"], None)
    assert rc == status


def test_sink_last_needs_an_entry_point_with_n_sink(lib):
    assert _fwd(lib, order=2) == -1
    # the counting entry points take it (validation passes up to the n_sink bound)
    rc = lib.fp8_attn_p_collapse_count(FAKE, FAKE, 1, 2, 1, 128, 128, 1, 2, 256.0, FAKE, FAKE, 65, FAKE, None)
    assert rc == -1


def test_decode_workspace_bytes(lib):
    assert lib.fp8_attn_decode_workspace_bytes(2, 4, 128, 8) == 2 * 4 * 8 * (128 + 4) * 4
    assert lib.fp8_attn_decode_workspace_bytes(1, 1, 96, 1) == 0
    assert lib.fp8_attn_decode_workspace_bytes(0, 1, 64, 1) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(ws=None), -1), (dict(n_split=0), -1),
    (dict(n_split=3), -1), (dict(ws_bytes=100), -1), (dict(order=2), -1), (dict(S=0.0), -1),
    (dict(H=3, Hkv=2), -1), (dict(d=80), -2), (dict(N=100), -2), (dict(ws=FAKE + 4), -2),
    (dict(q=FAKE + 8), -2),
])
def test_decode_validation(lib, kw, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, H=4, Hkv=2, N=128, d=128, order=1, S=256.0,
             qd=FAKE, kd=FAKE, vd=FAKE, n_split=2, ws=FAKE, ws_bytes=1 << 20)
    a.update(kw)
    rc = lib.fp8_attn_decode(a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["Hkv"], a["N"], a["d"],
                             a["order"], a["S"], a["qd"], a["kd"], a["vd"], a["n_split"], a["ws"], a["ws_bytes"],
                             None)
    assert rc == status


def test_binding_rejects_cpu_tensors():
    import torch

    x = torch.zeros((1, 1, 64, 64), dtype=torch.uint8)
    d = torch.ones(1, dtype=torch.float32)
    with pytest.raises(ValueError):
        binding.fwd(x, x, x, d, d, d, causal=False)


def test_product_path_does_not_import_the_oracle():
    """The HIP path and its binding never reference the CPU oracle."""
    pkg = os.path.join(ROOT, "precision_attention_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if path.endswith((".py", ".hip", ".h", ".cpp")):
            src = open(path).read()
            assert not re.search(r"^\s*(from\s+oracle\b|import\s+oracle\b)|\boracle\.", src, re.M), path


def test_binding_tensor_checks_on_cpu():
    """The binding's one check for every tensor it hands to the library refuses host
    tensors, wrong dtypes, shapes, element counts and short buffers (no GPU needed: the
    expected device is named, never touched)."""
    import torch

    dev = torch.device("cuda:0")
    ok_kw = dict(shape=(2, 3))
    with pytest.raises(ValueError, match="on cpu"):
        binding._check_tensor(torch.zeros(2, 3), "out", dev, torch.float32, **ok_kw)
    with pytest.raises(ValueError, match="expected a torch tensor"):
        binding._check_tensor([0.0] * 6, "out", dev, torch.float32, **ok_kw)
    meta = torch.empty(2, 3, device="meta")
    with pytest.raises(ValueError):
        binding._check_tensor(meta, "out", dev, torch.float32, **ok_kw)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), -1), (dict(ws_bytes=1), -1), (dict(d=256), -2), (dict(d=96), -2),
    (dict(order=3), -1), (dict(den=2), -1), (dict(n_sink=65, order=2), -1), (dict(ws=FAKE + 8), -2),
    (dict(S=449.0), -1), (dict(N=100), -2),
    # one head's bf16 keys (2 N d bytes) must fit a 32-bit buffer range: N = 2^23 at d = 128
    # is refused, N = 2^23 - 64 passes that check and fails on the small workspace
    (dict(N=1 << 23), -2), (dict(N=(1 << 23) - 64), -1),
])
def test_exact_qk_validation(lib, kw, status):
    a = dict(B=1, H=2, Hkv=1, N=128, d=128, causal=1, order=1, S=256.0, n_sink=4, den=0, ws=FAKE, ws_bytes=1 << 20)
    a.update(kw)
    rc = lib.fp8_attn_fwd_exact_qk(FAKE, FAKE, FAKE, FAKE, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["causal"],
                                   a["order"], a["S"], FAKE, FAKE, FAKE, a["n_sink"], a["den"], None, a["ws"],
                                   a["ws_bytes"], None)
    assert rc == status


def test_exact_qk_workspace_bytes(lib):
    assert lib.fp8_attn_fwd_exact_qk_workspace_bytes(2, 8, 4096, 128) == 2 * 8 * 4096 * 128 * 2
    assert lib.fp8_attn_fwd_exact_qk_workspace_bytes(1, 1, 64, 256) == 0


def test_decode_static_validation(lib):
    """fp8_attn_decode_static checks its arguments before any HIP call, and refuses split
    records beyond its static array (B=8, H=64, d=256, 64 splits: 34 MB > 8 MiB)."""
    call = lambda **kw: lib.fp8_attn_decode_static(
        kw.get("q", FAKE), FAKE, FAKE, FAKE, kw.get("B", 1), kw.get("H", 8), kw.get("Hkv", 2), kw.get("N", 4096),
        kw.get("d", 128), kw.get("order", 1), kw.get("S", 256.0), FAKE, FAKE, FAKE, kw.get("n_split", 8), None)
    assert call(q=None) == -1
    assert call(order=2) == -1
    assert call(n_split=0) == -1 and call(n_split=65) == -1
    assert call(d=96) == -2
    assert call(B=8, H=64, Hkv=64, N=64 * 64, d=256, n_split=64) == -4
    assert lib.fp8_attn_status_string(-4).startswith(b"request exceeds")


def _tile_rows(lib, B=1, H=8, Hkv=8, N=4096, d=128, causal=0, order=1, S=256.0, n_sink=4, den=0, exact=0):
    return lib.fp8_attn_fwd_tile_rows(B, H, Hkv, N, d, causal, order, S, n_sink, den, exact)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), -1), (dict(H=3, Hkv=2), -1), (dict(causal=2), -1), (dict(order=3), -1), (dict(S=0.0), -1),
    (dict(S=512.0), -1), (dict(n_sink=-1), -1), (dict(order=2, n_sink=65), -1), (dict(den=2), -1),
    (dict(exact=2), -1), (dict(d=96), -2), (dict(N=100), -2), (dict(d=256, exact=1), -2),
    (dict(N=1 << 23, d=128, exact=1), -2),
])
def test_tile_rows_validation(lib, kw, status):
    assert _tile_rows(lib, **kw) == status


@pytest.mark.parametrize("kw", [dict(d=64), dict(d=256), dict(order=2), dict(den=1), dict(exact=1)])
def test_tile_rows_32_without_consulting_the_device(lib, kw):
    # the 16-row kernel exists for d = 128 without the fwd_ex options or the exact Q.K^T only
    assert _tile_rows(lib, **kw) == 32


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), -1), (dict(H=3, Hkv=2), -1), (dict(causal=2), -1), (dict(order=3), -1), (dict(S=0.0), -1),
    (dict(S=512.0), -1), (dict(n_sink=-1), -1), (dict(order=2, n_sink=65), -1), (dict(den=2), -1),
    (dict(exact=2), -1), (dict(d=96), -2), (dict(N=100), -2), (dict(d=256, exact=1), -2),
    (dict(N=1 << 23, d=128, exact=1), -2),
])
def test_walk_groups_validation(lib, kw, status):
    # the same checks, and so the same statuses, as the tile-rows query
    assert _walk_groups(lib, **kw) == status == _tile_rows(lib, **kw)


@pytest.mark.parametrize("kw", [dict(d=64), dict(d=256), dict(order=2), dict(den=1), dict(exact=1)])
def test_walk_groups_1_without_consulting_the_device(lib, kw):
    # the two-group walk exists for d = 128 without the fwd_ex options or the exact Q.K^T only
    assert _walk_groups(lib, **kw) == 1


def _walk_groups(lib, B=1, H=8, Hkv=8, N=4096, d=128, causal=0, order=1, S=256.0, n_sink=4, den=0, exact=0):
    return lib.fp8_attn_fwd_walk_groups(B, H, Hkv, N, d, causal, order, S, n_sink, den, exact)


def test_decode_default_splits_rule():
    """About 512 waves (two per compute unit of MI355X), at least 8 blocks per split where N
    allows, never more splits than blocks."""
    from precision_attention_amd import binding

    assert binding.decode_default_splits(1, 8, 32, 131072) == 64      # 8 units x 64 = 512 waves
    assert binding.decode_default_splits(8, 8, 32, 32768) == 8        # 64 units x 8
    assert binding.decode_default_splits(1, 8, 32, 4096) == 8         # 64 blocks: 8 per split
    assert binding.decode_default_splits(1, 1, 1, 64) == 1            # one block
    assert binding.decode_default_splits(64, 8, 8, 32768) == 1        # 512 units need no split
    assert binding.decode_default_splits(1, 2, 80, 65536) == 128      # 2 KV heads x 3 query groups


def test_binding_static_scratch_size_matches_the_header():
    from precision_attention_amd import binding

    with open(os.path.join(ROOT, "include", "fp8attn.h")) as f:
        m = re.search(r"#define FP8ATTN_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and binding.STATIC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
