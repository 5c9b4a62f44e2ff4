"""Thin ctypes binding of the C ABI in include/fp8attn.h.

Argument marshalling only: shape/dtype/device checks, output allocation through torch
(device memory and streams are the only things torch provides), and a call into the
HIP library. Every step of the attention runs in the library's kernels. There is no
fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfp8attn.so")

FP8ATTN_OK = 0
STATIC_SCRATCH_BYTES = 8 << 20    # FP8ATTN_STATIC_SCRATCH_BYTES of include/fp8attn.h
KV_ORDERS = {"forward": 0, "reverse": 1, "reverse_sink_last": 2}
DENOMINATORS = {"fp32": 0, "quantized": 1}

_lib = None


def _declare(lib):
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fp8_attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp, vp]
    lib.fp8_attn_fwd.restype = i
    lib.fp8_attn_p_collapse_count.argtypes = [vp, vp, i, i, i, i, i, i, i, f, vp, vp, i, vp, vp]
    lib.fp8_attn_p_collapse_count.restype = i
    lib.fp8_attn_fwd_counted.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp, i, vp, vp]
    lib.fp8_attn_fwd_counted.restype = i
    lib.fp8_attn_fwd_ex.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp, i, i, vp, vp]
    lib.fp8_attn_fwd_ex.restype = i
    lib.fp8_attn_fwd_exact_qk_workspace_bytes.argtypes = [i, i, i, i]
    lib.fp8_attn_fwd_exact_qk_workspace_bytes.restype = ctypes.c_ulonglong
    lib.fp8_attn_fwd_exact_qk.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp, i, i, vp, vp,
                                          ctypes.c_ulonglong, vp]
    lib.fp8_attn_fwd_exact_qk.restype = i
    lib.fp8_attn_decode_workspace_bytes.argtypes = [i, i, i, i]
    lib.fp8_attn_decode_workspace_bytes.restype = ctypes.c_ulonglong
    lib.fp8_attn_decode.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, vp, i, vp, ctypes.c_ulonglong,
                                    vp]
    lib.fp8_attn_decode.restype = i
    lib.fp8_attn_decode_static.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, vp, i, vp]
    lib.fp8_attn_decode_static.restype = i
    lib.fp8_attn_fwd_tile_rows.argtypes = [i, i, i, i, i, i, i, f, i, i, i]
    lib.fp8_attn_fwd_tile_rows.restype = i
    lib.fp8_attn_fwd_walk_groups.argtypes = [i, i, i, i, i, i, i, f, i, i, i]
    lib.fp8_attn_fwd_walk_groups.restype = i
    lib.fp8_attn_kv_block.argtypes = []
    lib.fp8_attn_kv_block.restype = i
    lib.fp8_attn_version.argtypes = []
    lib.fp8_attn_version.restype = ctypes.c_char_p
    lib.fp8_attn_status_string.argtypes = [i]
    lib.fp8_attn_status_string.restype = ctypes.c_char_p


def load():
    """Load libfp8attn.so (built in-tree by ``build_lib.build()``); raise if missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(LIB_PATH)
        _declare(lib)
        _lib = lib
    return _lib


def _status(rc: int, what: str):
    if rc != FP8ATTN_OK:
        msg = load().fp8_attn_status_string(rc).decode()
        raise RuntimeError(f"{what} failed: status {rc} ({msg})")


def _as_codes(t, name):
    import torch

    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"{name}: expected uint8 E4M3 codes or float8_e4m3fn, got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous device tensor")
    return t


def _check_tensor(t, name, device, dtype, *, shape=None, numel=None, min_bytes=None):
    """Every tensor whose pointer reaches the library: a torch tensor, contiguous, on
    ``device`` (the GPU holding q), of ``dtype`` and of the required shape, element count
    or byte size. Raises ValueError before any library call otherwise."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, need at least {min_bytes}")
    return t


def _as_descale(t, n, name, device):
    import torch

    return _check_tensor(t, name, device, torch.float32, numel=n)


def _shapes(q8, k8, v8=None):
    for name, t in (("k", k8), ("v", v8)):
        if t is not None and t.device != q8.device:
            raise ValueError(f"{name}: on {t.device}, expected {q8.device} (the device of q)")
    if q8.dim() != 4 or k8.dim() != 4:
        raise ValueError("q and k must be [B, H, N, d] and [B, Hkv, N, d]")
    B, H, N, d = q8.shape
    Bk, Hkv, Nk, dk = k8.shape
    if (Bk, Nk, dk) != (B, N, d):
        raise ValueError(f"k shape {tuple(k8.shape)} does not match q {tuple(q8.shape)}")
    if v8 is not None and tuple(v8.shape) != tuple(k8.shape):
        raise ValueError(f"v shape {tuple(v8.shape)} differs from k {tuple(k8.shape)}")
    return B, H, Hkv, N, d


def _stream_ptr(device, stream):
    import torch

    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def fwd(q8, k8, v8, q_descale, k_descale, v_descale, *, causal: bool, kv_order: str = "reverse",
        S: float = 256.0, out=None, stream=None):
    """O = FP8 P-cast attention forward. q8 [B,H,N,d], k8/v8 [B,Hkv,N,d] E4M3 codes on the
    same GPU; descales float32 [B,H] / [B,Hkv]. Returns float32 [B,H,N,d] (``out`` if given).
    Enqueued on ``stream`` (default: the current stream); not synchronised."""
    import torch

    lib = load()
    q8, k8, v8 = _as_codes(q8, "q"), _as_codes(k8, "k"), _as_codes(v8, "v")
    B, H, Hkv, N, d = _shapes(q8, k8, v8)
    dev = q8.device
    qd = _as_descale(q_descale, B * H, "q_descale", dev)
    kd = _as_descale(k_descale, B * Hkv, "k_descale", dev)
    vd = _as_descale(v_descale, B * Hkv, "v_descale", dev)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    _check_tensor(out, "out", dev, torch.float32, shape=(B, H, N, d))
    rc = lib.fp8_attn_fwd(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                          B, H, Hkv, N, d, int(bool(causal)), KV_ORDERS[kv_order], float(S),
                          qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), _stream_ptr(dev, stream))
    _status(rc, "fp8_attn_fwd")
    return out


def p_collapse_count(q8, k8, q_descale, k_descale, *, causal: bool, kv_order: str = "reverse",
                     S: float = 256.0, n_sink: int = 4, out=None, stream=None):
    """Collapse counts (int64 [4] device tensor holding the library's uint64 counters):
    [collapsed non-sink P, of which in sink blocks, non-sink pairs, of which in sink blocks]."""
    import torch

    lib = load()
    q8, k8 = _as_codes(q8, "q"), _as_codes(k8, "k")
    B, H, Hkv, N, d = _shapes(q8, k8)
    dev = q8.device
    qd = _as_descale(q_descale, B * H, "q_descale", dev)
    kd = _as_descale(k_descale, B * Hkv, "k_descale", dev)
    if out is None:
        out = torch.empty(4, dtype=torch.int64, device=dev)
    _check_tensor(out, "out", dev, torch.int64, numel=4)
    rc = lib.fp8_attn_p_collapse_count(q8.data_ptr(), k8.data_ptr(), B, H, Hkv, N, d,
                                       int(bool(causal)), KV_ORDERS[kv_order], float(S),
                                       qd.data_ptr(), kd.data_ptr(), int(n_sink), out.data_ptr(),
                                       _stream_ptr(dev, stream))
    _status(rc, "fp8_attn_p_collapse_count")
    return out


def fwd_counted(q8, k8, v8, q_descale, k_descale, v_descale, *, causal: bool, kv_order: str = "reverse",
                S: float = 256.0, n_sink: int = 4, out=None, counts=None, stream=None):
    """Forward pass and collapse counts in one launch. Returns (O, counts) with the same
    meaning as ``fwd`` and ``p_collapse_count``."""
    import torch

    lib = load()
    q8, k8, v8 = _as_codes(q8, "q"), _as_codes(k8, "k"), _as_codes(v8, "v")
    B, H, Hkv, N, d = _shapes(q8, k8, v8)
    dev = q8.device
    qd = _as_descale(q_descale, B * H, "q_descale", dev)
    kd = _as_descale(k_descale, B * Hkv, "k_descale", dev)
    vd = _as_descale(v_descale, B * Hkv, "v_descale", dev)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    _check_tensor(out, "out", dev, torch.float32, shape=(B, H, N, d))
    if counts is None:
        counts = torch.empty(4, dtype=torch.int64, device=dev)
    _check_tensor(counts, "counts", dev, torch.int64, numel=4)
    rc = lib.fp8_attn_fwd_counted(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                                  B, H, Hkv, N, d, int(bool(causal)), KV_ORDERS[kv_order], float(S),
                                  qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), int(n_sink), counts.data_ptr(),
                                  _stream_ptr(dev, stream))
    _status(rc, "fp8_attn_fwd_counted")
    return out, counts


def fwd_ex(q8, k8, v8, q_descale, k_descale, v_descale, *, causal: bool, kv_order: str = "reverse",
           S: float = 256.0, n_sink: int = 4, denominator: str = "fp32", count: bool = False,
           out=None, counts=None, stream=None):
    """The forward with every option: ``kv_order`` also "reverse_sink_last" (block 0's
    non-sink keys visited before the n_sink sink tokens), ``denominator`` "fp32" (row sum
    of P~ S) or "quantized" (row sum of the decoded E4M3 P). With ``count`` (or a
    ``counts`` tensor) the collapse counts are filled too. Returns (O, counts or None)."""
    import torch

    lib = load()
    q8, k8, v8 = _as_codes(q8, "q"), _as_codes(k8, "k"), _as_codes(v8, "v")
    B, H, Hkv, N, d = _shapes(q8, k8, v8)
    dev = q8.device
    qd = _as_descale(q_descale, B * H, "q_descale", dev)
    kd = _as_descale(k_descale, B * Hkv, "k_descale", dev)
    vd = _as_descale(v_descale, B * Hkv, "v_descale", dev)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    _check_tensor(out, "out", dev, torch.float32, shape=(B, H, N, d))
    if counts is None and count:
        counts = torch.empty(4, dtype=torch.int64, device=dev)
    if counts is not None:
        _check_tensor(counts, "counts", dev, torch.int64, numel=4)
    rc = lib.fp8_attn_fwd_ex(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                             B, H, Hkv, N, d, int(bool(causal)), KV_ORDERS[kv_order], float(S),
                             qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), int(n_sink), DENOMINATORS[denominator],
                             None if counts is None else counts.data_ptr(), _stream_ptr(dev, stream))
    _status(rc, "fp8_attn_fwd_ex")
    return out, counts


def fwd_exact_qk(q8, k8, v8, q_descale, k_descale, v_descale, *, causal: bool, kv_order: str = "reverse",
                 S: float = 256.0, n_sink: int = 4, denominator: str = "fp32", count: bool = False,
                 out=None, counts=None, workspace=None, stream=None):
    """``fwd_ex`` with Q.K^T from exact products accumulated in fp32 (bf16 matrix cores),
    d 64 or 128. ``workspace`` (optional): a uint8 device tensor of at least
    ``fp8_attn_fwd_exact_qk_workspace_bytes`` bytes. Returns (O, counts or None)."""
    import torch

    lib = load()
    q8, k8, v8 = _as_codes(q8, "q"), _as_codes(k8, "k"), _as_codes(v8, "v")
    B, H, Hkv, N, d = _shapes(q8, k8, v8)
    dev = q8.device
    qd = _as_descale(q_descale, B * H, "q_descale", dev)
    kd = _as_descale(k_descale, B * Hkv, "k_descale", dev)
    vd = _as_descale(v_descale, B * Hkv, "v_descale", dev)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    _check_tensor(out, "out", dev, torch.float32, shape=(B, H, N, d))
    if counts is None and count:
        counts = torch.empty(4, dtype=torch.int64, device=dev)
    if counts is not None:
        _check_tensor(counts, "counts", dev, torch.int64, numel=4)
    need = int(lib.fp8_attn_fwd_exact_qk_workspace_bytes(B, Hkv, N, d))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check_tensor(workspace, "workspace", dev, torch.uint8, min_bytes=need)
    rc = lib.fp8_attn_fwd_exact_qk(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                                   B, H, Hkv, N, d, int(bool(causal)), KV_ORDERS[kv_order], float(S),
                                   qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), int(n_sink),
                                   DENOMINATORS[denominator], None if counts is None else counts.data_ptr(),
                                   workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream_ptr(dev, stream))
    _status(rc, "fp8_attn_fwd_exact_qk")
    return out, counts


def decode_default_splits(B: int, Hkv: int, H: int, N: int, target_waves: int = 512,
                          min_blocks_per_split: int = 8) -> int:
    """Split count for fp8_attn_decode: enough splits for about ``target_waves`` waves in
    the grid, two per compute unit of MI355X (one wave per (batch, KV head, group of up to 32
    query heads, split)). Measured on MI355X for 1 sequence of 128K keys and 8 of 32K: one
    wave per compute unit leaves the stream latency-bound (4.3-4.5 TB/s), four lose HBM
    efficiency to the extra concurrent streams. Splits keep at least
    ``min_blocks_per_split`` 64-key blocks where the sequence allows it, so that the per-split
    start-up and the merge stay small."""
    nb = N // 64
    units = B * Hkv * ((H // Hkv + 31) // 32)
    n = -(-target_waves // units)
    n = min(n, max(1, nb // min_blocks_per_split))
    return max(1, min(nb, n))


def decode(q8, k8, v8, q_descale, k_descale, v_descale, *, kv_order: str = "reverse", S: float = 256.0,
           n_split: int | None = None, out=None, workspace=None, stream=None):
    """Split-KV decode: q8 [B,H,d] (one query row per head), k8/v8 [B,Hkv,N,d] E4M3 codes;
    every query sees all N keys. Returns float32 [B,H,d]. ``workspace`` (optional) is a
    uint8 device tensor of at least ``fp8_attn_decode_workspace_bytes`` bytes."""
    import torch

    lib = load()
    q8, k8, v8 = _as_codes(q8, "q"), _as_codes(k8, "k"), _as_codes(v8, "v")
    if q8.dim() != 3 or k8.dim() != 4 or tuple(v8.shape) != tuple(k8.shape):
        raise ValueError("q must be [B, H, d], k and v [B, Hkv, N, d]")
    B, H, d = q8.shape
    Bk, Hkv, N, dk = k8.shape
    if (Bk, dk) != (B, d):
        raise ValueError(f"k shape {tuple(k8.shape)} does not match q {tuple(q8.shape)}")
    dev = q8.device
    for name, t in (("k", k8), ("v", v8)):
        if t.device != dev:
            raise ValueError(f"{name}: on {t.device}, expected {dev} (the device of q)")
    qd = _as_descale(q_descale, B * H, "q_descale", dev)
    kd = _as_descale(k_descale, B * Hkv, "k_descale", dev)
    vd = _as_descale(v_descale, B * Hkv, "v_descale", dev)
    if n_split is None:
        n_split = decode_default_splits(B, Hkv, H, N)
    need = lib.fp8_attn_decode_workspace_bytes(B, H, d, int(n_split))
    if workspace is None:
        workspace = torch.empty(max(int(need), 16), dtype=torch.uint8, device=dev)
    _check_tensor(workspace, "workspace", dev, torch.uint8, min_bytes=int(need))
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    _check_tensor(out, "out", dev, torch.float32, shape=(B, H, d))
    rc = lib.fp8_attn_decode(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(), B, H, Hkv, N, d,
                             KV_ORDERS[kv_order], float(S), qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                             int(n_split), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                             _stream_ptr(dev, stream))
    _status(rc, "fp8_attn_decode")
    return out


def decode_static(q8, k8, v8, q_descale, k_descale, v_descale, *, kv_order: str = "reverse", S: float = 256.0,
                  n_split: int | None = None, out=None, stream=None):
    """``decode`` with the split records in the library's static per-GPU scratch
    (fp8_attn_decode_static: no workspace; calls overlapping on one GPU race). Without
    ``n_split``, the default split count is lowered to what the scratch holds."""
    import torch

    lib = load()
    q8, k8, v8 = _as_codes(q8, "q"), _as_codes(k8, "k"), _as_codes(v8, "v")
    if q8.dim() != 3 or k8.dim() != 4 or tuple(v8.shape) != tuple(k8.shape):
        raise ValueError("q must be [B, H, d], k and v [B, Hkv, N, d]")
    B, H, d = q8.shape
    Bk, Hkv, N, dk = k8.shape
    if (Bk, dk) != (B, d):
        raise ValueError(f"k shape {tuple(k8.shape)} does not match q {tuple(q8.shape)}")
    dev = q8.device
    for name, t in (("k", k8), ("v", v8)):
        if t.device != dev:
            raise ValueError(f"{name}: on {t.device}, expected {dev} (the device of q)")
    qd = _as_descale(q_descale, B * H, "q_descale", dev)
    kd = _as_descale(k_descale, B * Hkv, "k_descale", dev)
    vd = _as_descale(v_descale, B * Hkv, "v_descale", dev)
    if n_split is None:
        per_split = lib.fp8_attn_decode_workspace_bytes(B, H, d, 1)
        fit = STATIC_SCRATCH_BYTES // per_split if per_split else 1
        n_split = max(1, min(decode_default_splits(B, Hkv, H, N), fit))
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    _check_tensor(out, "out", dev, torch.float32, shape=(B, H, d))
    rc = lib.fp8_attn_decode_static(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(), B, H, Hkv, N, d,
                                    KV_ORDERS[kv_order], float(S), qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                                    int(n_split), _stream_ptr(dev, stream))
    _status(rc, "fp8_attn_decode_static")
    return out


def fwd_tile_rows(B, H, Hkv, N, d, *, causal=True, kv_order="reverse", S=256.0, n_sink=4,
                  denominator="fp32", exact_qk=False) -> int:
    """Query rows per wave (16 or 32) the forward entry points use for these arguments on
    the current device (fp8_attn_fwd_tile_rows)."""
    rc = load().fp8_attn_fwd_tile_rows(B, H, Hkv, N, d, int(bool(causal)), KV_ORDERS[kv_order], float(S),
                                       int(n_sink), DENOMINATORS[denominator], int(bool(exact_qk)))
    if rc < 0:
        _status(rc, "fp8_attn_fwd_tile_rows")
    return rc


def fwd_walk_groups(B, H, Hkv, N, d, *, causal=True, kv_order="reverse", S=256.0, n_sink=4,
                    denominator="fp32", exact_qk=False) -> int:
    """Walk groups (1, or 2: 64-row tiles whose KV walk two groups of waves split) the
    32-row forward uses for these arguments on the current device
    (fp8_attn_fwd_walk_groups)."""
    rc = load().fp8_attn_fwd_walk_groups(B, H, Hkv, N, d, int(bool(causal)), KV_ORDERS[kv_order], float(S),
                                         int(n_sink), DENOMINATORS[denominator], int(bool(exact_qk)))
    if rc < 0:
        _status(rc, "fp8_attn_fwd_walk_groups")
    return rc


def kv_block() -> int:
    return load().fp8_attn_kv_block()


def version() -> str:
    return load().fp8_attn_version().decode()
