"""Seeded synthetic inputs for the FP8 P-cast attention forward.

This module is shared by the tests, the benchmark and the smoke check. It holds none
of the method's arithmetic: it draws Gaussian (or Student-t) Q, K, V, plants the
attention sink, and quantizes to E4M3 with torch's own float8_e4m3fn cast (a library
routine) after clamping to the finite range. It imports neither the oracle nor the
HIP library.

Sink construction. The P-Cast pages define the sink strength Δ as the logit gap
between sink and non-sink tokens, with k = 4 sink tokens and non-sink logits standard
normal (P-Cast technical summary, §2 Theoretical framework). The synthetic recipe:
  * Q, K, V ~ N(0, 1) (V optionally Student-t with 4 degrees of freedom), float32;
  * alpha = sqrt(Δ·sqrt(d)); column 0 of every query row is alpha and column 0 of the
    first ``n_sink`` keys is alpha, so a sink logit is Δ + N(0, (d-1)/d);
  * "clean" (default): column 0 of every other key is 0, so non-sink logits are
    N(0, (d-1)/d), the closed form's premise; "literal": those entries stay N(0, 1);
  * E4M3 quantization with descale = amax/448 per tensor or per (batch, head).
Sinks are planted in every KV head and the sink column in every query head.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

E4M3_FINITE_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    """One synthetic attention workload (sizes, mask, sink, value law, descale)."""
    name: str
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    causal: bool
    delta: float
    orders: tuple = ("reverse",)
    scales: tuple = (256.0,)
    n_sink: int = 4
    v_dist: str = "normal"
    descale: str = "head"
    deltas: tuple = field(default_factory=tuple)
    decode: bool = False          # one query row per head (the last position), all N keys

    def flop(self) -> float:
        """Algorithmic FLOP: 2 GEMMs x 2·d per unmasked (query, key) pair."""
        if self.decode:
            return 4.0 * self.d * self.B * self.H * self.N
        pairs = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return 4.0 * self.d * self.B * self.H * pairs

    def bytes(self) -> float:
        """Algorithmic bytes: Q, K, V once (1 B per element) and O once (4 B per element)."""
        nq = 1 if self.decode else self.N
        return float(self.B * self.d * (self.H * nq * (1 + 4) + 2 * self.Hkv * self.N))


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_noncausal_n1024_d64", 1, 1, 1, 1024, 64, False, 8.0,
                 orders=("forward", "reverse"), scales=(1.0, 256.0), descale="tensor"),
        Workload("sweep_noncausal_h8_n4096_d128", 1, 8, 8, 4096, 128, False, 8.0,
                 orders=("forward", "reverse"), scales=(1.0, 16.0, 256.0, 448.0),
                 descale="tensor", deltas=(0.0, 4.0, 6.0, 7.0, 8.0, 10.0, 12.0)),
        Workload("causal_b4_h32_n8192_d128", 4, 32, 32, 8192, 128, True, 8.0,
                 orders=("reverse", "forward"), scales=(256.0,), descale="head"),
        Workload("causal_h4_n8192_d128", 1, 4, 4, 8192, 128, True, 8.0,
                 orders=("reverse",), scales=(256.0,), descale="head"),
        Workload("gqa_causal_h32_kv8_n32768_d128", 1, 32, 8, 32768, 128, True, 10.0,
                 orders=("reverse", "forward"), scales=(256.0,), descale="head"),
        Workload("causal_h16_n65536_d128", 1, 16, 16, 65536, 128, True, 12.0,
                 orders=("reverse",), scales=(256.0,), v_dist="student_t4", descale="head"),
        Workload("causal_h16_n65536_d256", 1, 16, 16, 65536, 256, True, 12.0,
                 orders=("reverse",), scales=(256.0,), v_dist="student_t4", descale="head"),
        Workload("decode_gqa_h32_kv8_n131072_d128", 1, 32, 8, 131072, 128, False, 10.0,
                 orders=("reverse", "forward"), scales=(256.0,), descale="head", decode=True),
        Workload("decode_b8_gqa_h32_kv8_n32768_d128", 8, 32, 8, 32768, 128, False, 10.0,
                 orders=("reverse",), scales=(256.0,), descale="head", decode=True),
    ]
}


def sink_alpha(delta: float, d: int) -> float:
    """Sink column value: alpha^2/sqrt(d) = Δ."""
    return math.sqrt(max(delta, 0.0) * math.sqrt(d))


def quantize_e4m3(x: np.ndarray, per: str):
    """E4M3 bytes and fp32 descales (amax/448) of a [B, H, N, d] float32 array.

    ``per`` = "tensor" (one descale broadcast to every (b, h)) or "head".
    Returns (codes uint8 [B, H, N, d], descale float32 [B, H]).
    """
    import torch

    B, H = x.shape[:2]
    if per == "tensor":
        amax = np.full((B, H), np.abs(x).max(), dtype=np.float32)
    elif per == "head":
        amax = np.abs(x).reshape(B, H, -1).max(axis=2).astype(np.float32)
    else:
        raise ValueError(per)
    amax = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    descale = (amax / np.float32(E4M3_FINITE_MAX)).astype(np.float32)
    scaled = x / descale[:, :, None, None]
    np.clip(scaled, -E4M3_FINITE_MAX, E4M3_FINITE_MAX, out=scaled)
    codes = torch.from_numpy(np.ascontiguousarray(scaled)).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8).numpy(), descale


def make_inputs(B: int, H: int, Hkv: int, N: int, d: int, *, delta: float, n_sink: int = 4,
                seed: int = 0, construction: str = "clean", v_dist: str = "normal",
                descale: str = "head", keep_float: bool = True, n_q: int | None = None):
    """Draw one seeded input set. Random draws: PCG64 ``default_rng(seed)``, Q then K
    then V, each as float32 ``standard_normal`` (V: ``standard_t(4)`` cast to float32).

    Returns a dict with uint8 ``q8`` [B,H,n_q,d] (n_q = N unless given: decode draws one
    query position), ``k8``/``v8`` [B,Hkv,N,d], float32 descales ``qd`` [B,H],
    ``kd``/``vd`` [B,Hkv] and, if ``keep_float``, the float32 sources ``q``, ``k``, ``v``
    (after the sink is planted, before quantization).
    """
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N if n_q is None else n_q, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    if v_dist == "normal":
        v = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    elif v_dist == "student_t4":
        v = rng.standard_t(4, size=(B, Hkv, N, d)).astype(np.float32)
    else:
        raise ValueError(v_dist)
    a = np.float32(sink_alpha(delta, d))
    q[..., 0] = a
    k[:, :, :n_sink, 0] = a
    if construction == "clean":
        k[:, :, n_sink:, 0] = 0.0
    elif construction != "literal":
        raise ValueError(construction)
    q8, qd = quantize_e4m3(q, descale)
    k8, kd = quantize_e4m3(k, descale)
    v8, vd = quantize_e4m3(v, descale)
    out = {"q8": q8, "k8": k8, "v8": v8, "qd": qd, "kd": kd, "vd": vd}
    if keep_float:
        out.update(q=q, k=k, v=v)
    return out


def make_workload_inputs(w: Workload, *, seed: int = 0, delta: float | None = None,
                         construction: str = "clean", keep_float: bool = True):
    """``make_inputs`` with a workload's sizes and sink/value/descale recipe."""
    inp = make_inputs(w.B, w.H, w.Hkv, w.N, w.d, delta=w.delta if delta is None else delta,
                      n_sink=w.n_sink, seed=seed, construction=construction,
                      v_dist=w.v_dist, descale=w.descale, keep_float=keep_float,
                      n_q=1 if w.decode else None)
    if w.decode:                  # q [B, H, d]: the single query position
        for key in ("q8", "q"):
            if key in inp:
                inp[key] = np.ascontiguousarray(inp[key][:, :, 0, :])
    return inp


def sample_rows(N: int, n_rows: int, seed: int = 0, edge: int = 128):
    """Row subset for full-size checks: the first and last ``edge`` rows plus seeded
    random rows (sorted, unique)."""
    rng = np.random.default_rng(10_000 + seed)
    edge = min(edge, N // 2)
    fixed = np.concatenate([np.arange(edge), np.arange(N - edge, N)])
    extra = max(n_rows - len(fixed), 0)
    rest = rng.choice(np.arange(edge, N - edge), size=min(extra, N - 2 * edge), replace=False)
    return np.unique(np.concatenate([fixed, rest]))
