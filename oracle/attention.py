"""fp64 oracle of the FP8 P-cast attention forward (online softmax, block order, S).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What it computes, and where the pages fix it
--------------------------------------------
P-Cast technical summary ("P-Cast Precision in FP8 Attention", gist.science):
  * §1 Problem statement: Q·K^T and P·V run on FP8 (E4M3) operands; the softmax
    probabilities P are cast to E4M3 before the P·V product; an online softmax keeps a
    running maximum m over the KV blocks, so a large sink logit raises m and pushes the
    later non-sink P towards zero ("P-collapse").
  * §1, the two implementation choices: the KV block order (forward 0->N or reverse
    N->0) and a static scale S multiplied onto P before the cast and divided back out
    in the epilogue.
  * §2 Optimization 2, condition 1: for S = 2^k the multiply and divide are exact.
EFQ-Softmax abstract ("EFQ-Softmax: Exp-Free Quantization for Softmax"): the
conventional low-bit path evaluates the shifted exponentials in high precision, forms
the probability block, then quantizes it for the low-bit P·V product; the row-max
update, the rescale of the history, high-precision accumulation and the final
normalisation are the usual FlashAttention steps.

Readings taken where the pages leave a step open (each is listed in the design notes):
  * the logits are natural-log units with the usual 1/sqrt(d) scale;
  * KV blocks are 64 keys wide, aligned at key 0; the running max is updated exactly
    once per block, starting from -inf;
  * the row sum l accumulates the *unquantized* P~ = exp(s - m); only the operand of
    P·V is scaled and cast (the pages apply S and the cast "before the P·V product");
  * the cast is E4M3FN round-to-nearest-even of the fp64 product P~·S;
  * O = acc / (S·l) once, in the epilogue;
  * causal masking is j <= i with equal query and key lengths; a block that is
    entirely masked for a row leaves that row's state unchanged.

Two variants beyond the pages' own two choices (order, S), each an option here:
  * "reverse_sink_last": the reverse walk with block 0 split in two visits, its non-sink
    keys [n_sink, 64) first and the sink keys [0, n_sink) last. It applies the pages'
    reason for the reverse order (§2, Optimization 1: the sink should raise m only after
    every other P has been cast) to the tokens that share block 0 with the sinks.
  * denominator "quantized": l accumulates the decoded cast operand dec(P8) instead of
    P~·S, so that the same quantized P feeds the numerator and the denominator (the
    consistency idea of the EFQ-Softmax abstract, applied to the E4M3 cast); then
    O = acc / l.
And one more workload shape: decode (one query row per head over all N keys) with the key
range split into contiguous ranges. Each split runs the recurrence above on its own keys
(its own running max, its blocks in the chosen order), and the split states are merged
exactly through their maxima, as FlashAttention-style split-KV does. The P cast therefore
depends on the split, and the oracle reproduces that partition.

Everything is fp64. Q·K^T is taken over the raw decoded E4M3 values, which is exact
in fp64 (every product is a multiple of 2^-18 and every partial sum stays far below
2^53 of those units), and the descales are applied afterwards.
"""
from __future__ import annotations

import math

import numpy as np

from . import e4m3, mfma_model

BLOCK = 64
N_SINK_DEFAULT = 4
FLIP_REL_WINDOW = 2.0 ** -16      # relative half-width of the rounding-boundary band


# --------------------------------------------------------------------------------------
# inputs
# --------------------------------------------------------------------------------------

def head_logits_e4m3(q8, k8, qd: float, kd: float, d: int, rows=None, causal=False):
    """Natural-log logits s = (dec(Q8)·dec(K8)^T)·qd·kd/sqrt(d) for one head, fp64.

    ``q8``: [N, d] uint8, ``k8``: [N, d] uint8. ``rows``: optional query row indices.
    Masked entries (causal, j > i) are -inf.
    """
    qv = e4m3.decode(q8)
    kv = e4m3.decode(k8)
    idx = np.arange(qv.shape[0]) if rows is None else np.asarray(rows)
    raw = qv[idx] @ kv.T                        # exact: see module docstring
    s = raw * (float(qd) * float(kd)) / math.sqrt(d)
    if causal:
        s = np.where(np.arange(kv.shape[0])[None, :] > idx[:, None], -np.inf, s)
    return s, idx


def head_logits_float(q, k, d: int, rows=None, causal=False):
    """Logits from real-valued Q, K (the "Q, K, V kept in fp32" simulation mode)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = (q[idx] @ k.T) / math.sqrt(d)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > idx[:, None], -np.inf, s)
    return s, idx


def block_visit_order(n_keys: int, kv_order: str, block: int = BLOCK):
    """Block indices in visit order: forward 0..nb-1 or reverse nb-1..0.

    With causal masking a block past a row's diagonal is fully masked for that row
    and is a no-op, so row i effectively visits 0..floor(i/64) (forward) or
    floor(i/64)..0 (reverse): the reverse walk starts at the diagonal block.
    """
    nb = n_keys // block
    if kv_order == "forward":
        return list(range(nb))
    if kv_order in ("reverse", "reverse_sink_last"):
        return list(range(nb - 1, -1, -1))
    raise ValueError(kv_order)


def visit_units(n_keys: int, kv_order: str, block: int = BLOCK, n_sink: int = N_SINK_DEFAULT):
    """The key ranges [start, end) in visit order; each range is one online-softmax step
    (one running-max update). For "forward" and "reverse" they are the blocks. For
    "reverse_sink_last" block 0 is visited as [n_sink, 64) and then [0, n_sink) (empty
    ranges dropped; needs 0 <= n_sink <= block)."""
    units = [(b * block, (b + 1) * block) for b in block_visit_order(n_keys, kv_order, block)]
    if kv_order == "reverse_sink_last" and units:
        if not 0 <= n_sink <= block:
            raise ValueError("reverse_sink_last needs 0 <= n_sink <= block")
        units = units[:-1] + [u for u in ((n_sink, block), (0, n_sink)) if u[1] > u[0]]
    return units


# --------------------------------------------------------------------------------------
# the online-softmax P-cast forward, block by block (the method's own order)
# --------------------------------------------------------------------------------------

def _cast(p_scaled, p_cast: str):
    if p_cast == "e4m3":
        return e4m3.round_e4m3(p_scaled)
    if p_cast == "bf16":
        return e4m3.round_bf16(p_scaled)
    if p_cast == "none":
        return p_scaled
    raise ValueError(p_cast)


def online_softmax_pcast(s, v, *, kv_order: str, S: float, p_cast: str = "e4m3",
                         block: int = BLOCK, keep_trace: bool = False, n_sink: int = N_SINK_DEFAULT,
                         denominator: str = "fp32"):
    """Run the block-wise online softmax with the P-cast for a set of rows.

    ``s``: [R, N] fp64 logits (-inf where masked). ``v``: [N, d] fp64 values (already
    multiplied by their descale). For each row, the key ranges of ``visit_units`` are
    visited in order (the blocks, for forward and reverse); per range:
        m_new = max(m, max_j s_ij)
        alpha = exp(m - m_new)                     (0 while m = -inf)
        P~_ij = exp(s_ij - m_new)
        P8_ij = cast(P~_ij · S)
        l     = alpha·l + sum_j P~_ij·S            (denominator "fp32": unquantized P~)
          or  = alpha·l + sum_j P8_ij              (denominator "quantized")
        acc   = alpha·acc + sum_j P8_ij · v_j
        m     = m_new
    and O = acc / l. (With "fp32", l carries the factor S, i.e. O = acc / (S · sum P~).)
    Rows are processed together but every row follows exactly its own sequence; a range
    with no unmasked key for a row changes nothing for it.

    Returns (O [R, d], trace) where ``trace`` (if requested) holds, per visited range,
    its bounds, m after it, P~ and the cast operand P8.
    """
    if denominator not in ("fp32", "quantized"):
        raise ValueError(denominator)
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    R, N = s.shape
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, v.shape[1]))
    trace = []
    for (j0, j1) in visit_units(N, kv_order, block, n_sink):
        sb = s[:, j0:j1]
        live = np.isfinite(sb)                               # unmasked entries
        row_live = live.any(axis=1)
        bmax = np.where(live, sb, -np.inf).max(axis=1)
        m_new = np.where(row_live, np.maximum(m, bmax), m)
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
            p = np.where(live, np.exp(sb - m_new[:, None]), 0.0)
        p8 = _cast(p * S, p_cast)
        l = alpha * l + (p.sum(axis=1) * S if denominator == "fp32" else p8.sum(axis=1))
        acc = alpha[:, None] * acc + p8 @ v[j0:j1]
        m = m_new
        if keep_trace:
            trace.append({"block": j0 // block, "range": (j0, j1), "m": m.copy(), "p": p, "p8": p8,
                          "live": live})
    o = acc / l[:, None]
    return o, trace


def _running_max_at_key(s, kv_order, block, n_sink=N_SINK_DEFAULT):
    """m_u(i) at every key: row i's running max right after visiting the range that holds
    key j, and the final max m_f(i)."""
    R, N = s.shape
    fin = np.where(np.isfinite(s), s, -np.inf)
    m_at_key = np.full((R, N), -np.inf)
    cur = np.full(R, -np.inf)
    for (j0, j1) in visit_units(N, kv_order, block, n_sink):
        cur = np.maximum(cur, fin[:, j0:j1].max(axis=1))
        m_at_key[:, j0:j1] = cur[:, None]
    return m_at_key, cur


def online_softmax_pcast_vectorized(s, v, *, kv_order: str, S: float, p_cast: str = "e4m3",
                                    block: int = BLOCK, n_sink: int = N_SINK_DEFAULT,
                                    denominator: str = "fp32"):
    """The same result written in closed form instead of as a recurrence.

    Let m_u(i) be row i's running max right after visiting range u and m_f(i) the final
    max. Unrolling the recurrence, range u's contribution is rescaled by every later
    alpha, i.e. by exp(m_u - m_f), and the row sum telescopes:

        O_i = sum_j cast(exp(s_ij - m_u(j)(i))·S)·exp(m_u(j)(i) - m_f(i))·v_j / L_i
        L_i = S · sum_j exp(s_ij - m_f(i))                                ("fp32")
            = sum_j cast(exp(s_ij - m_u(j)(i))·S)·exp(m_u(j)(i) - m_f(i))  ("quantized")

    where u(j) is the range holding key j. Equal to the recurrence in real arithmetic.
    """
    s = np.asarray(s, dtype=np.float64)
    m_at_key, m_f = _running_max_at_key(s, kv_order, block, n_sink)
    live = np.isfinite(s)
    with np.errstate(invalid="ignore"):
        p = np.where(live, np.exp(s - m_at_key), 0.0)
        w = np.where(live, np.exp(m_at_key - m_f[:, None]), 0.0)
        l = np.where(live, np.exp(s - m_f[:, None]), 0.0).sum(axis=1) * S
    p8 = _cast(p * S, p_cast)
    if denominator == "quantized":
        l = (p8 * w).sum(axis=1)
    elif denominator != "fp32":
        raise ValueError(denominator)
    return ((p8 * w) @ np.asarray(v, dtype=np.float64)) / l[:, None]


def exact_attention(s, v):
    """Plain softmax(s)·v in fp64 (no cast): the exact attention the cast perturbs."""
    s = np.asarray(s, dtype=np.float64)
    mx = np.where(np.isfinite(s), s, -np.inf).max(axis=1, keepdims=True)
    e = np.where(np.isfinite(s), np.exp(s - mx), 0.0)
    return (e / e.sum(axis=1, keepdims=True)) @ np.asarray(v, dtype=np.float64)


# --------------------------------------------------------------------------------------
# P-collapse diagnostic
# --------------------------------------------------------------------------------------

def collapse_counts(s, *, kv_order: str, S: float, n_sink: int = N_SINK_DEFAULT,
                    block: int = BLOCK, row_ids=None):
    """Counts of collapsed non-sink probabilities for a set of rows.

    A probability collapses when its cast operand is the E4M3 zero although the key is
    unmasked (P-Cast summary, §1: non-sink P underflows to zero under the inflated
    running max). Only non-sink keys j >= n_sink are counted. Returns a length-4
    integer vector:
        [0] collapsed non-sink P over all blocks
        [1] of which in blocks that contain a sink key (64·b < n_sink)
        [2] unmasked non-sink (i, j) pairs over all blocks
        [3] of which in blocks that contain a sink key
    The cast operand is computed exactly as in ``online_softmax_pcast``; "blocks that
    contain a sink key" are the 64-key blocks, also when "reverse_sink_last" visits
    block 0 in two ranges.
    """
    s = np.asarray(s, dtype=np.float64)
    R, N = s.shape
    out = np.zeros(4, dtype=np.int64)
    m = np.full(R, -np.inf)
    keys = np.arange(N)
    for (j0, j1) in visit_units(N, kv_order, block, n_sink):
        sb = s[:, j0:j1]
        live = np.isfinite(sb)
        row_live = live.any(axis=1)
        bmax = np.where(live, sb, -np.inf).max(axis=1)
        m = np.where(row_live, np.maximum(m, bmax), m)
        with np.errstate(invalid="ignore"):
            p = np.where(live, np.exp(sb - m[:, None]), 0.0)
        code = e4m3.encode(p * S)
        nonsink = (keys[j0:j1] >= n_sink)[None, :]
        counted = live & nonsink
        zero = counted & (code == 0)
        sink_block = (j0 // block) * block < n_sink
        out[0] += int(zero.sum())
        out[2] += int(counted.sum())
        if sink_block:
            out[1] += int(zero.sum())
            out[3] += int(counted.sum())
    return out


def collapse_count_slack(s, *, kv_order: str, S: float, s_err=None, n_sink: int = N_SINK_DEFAULT,
                         block: int = BLOCK):
    """How far a device's collapse count may legitimately differ from ``collapse_counts``:
    the counted (unmasked, non-sink) pairs whose cast operand could land on either side of
    the zero boundary 2^-10 (E4M3 rounds x <= 2^-10 to zero), given the relative fp32 band
    FLIP_REL_WINDOW around P~·S and, with ``s_err``, the logit interval of the device's Q·K^T
    (the same interval as ``flip_allowance``). Returns [all blocks, blocks holding a sink]."""
    s = np.asarray(s, dtype=np.float64)
    live = np.isfinite(s)
    m_at_key, _ = _running_max_at_key(s, kv_order, block, n_sink)
    if s_err is None:
        spread = np.zeros_like(s)
    else:
        e_ij = np.where(live, np.asarray(s_err, dtype=np.float64), 0.0)
        e_run, _ = _running_max_at_key(np.where(live, e_ij, -np.inf), kv_order, block, n_sink)
        spread = e_ij + np.where(np.isfinite(e_run), e_run, 0.0)
    with np.errstate(invalid="ignore", over="ignore"):
        x = np.where(live, np.exp(s - m_at_key) * S, 0.0)
    zero = 2.0 ** -10
    both = (x * np.exp(-spread) * (1.0 - FLIP_REL_WINDOW) <= zero) & (x * np.exp(spread) * (1.0 + FLIP_REL_WINDOW) > zero)
    keys = np.arange(s.shape[1])
    counted = live & (keys >= n_sink)[None, :] & both
    sink_cols = keys < ((n_sink + block - 1) // block) * block
    return np.array([int(counted.sum()), int(counted[:, sink_cols].sum())], dtype=np.int64)


# --------------------------------------------------------------------------------------
# rounding-boundary allowance
# --------------------------------------------------------------------------------------

def _e4m3_boundaries():
    vals = e4m3.all_finite_values()
    mids = (vals[:-1] + vals[1:]) / 2.0          # rounding midpoints; mids[0] = 2^-10
    return vals, mids


def _allowance_from(s, v, m_at_key, e_ij, e_run, *, S: float, denominator: str):
    """The output tolerance of one set of rows, given for every (i, j) the exact running max
    m_u(j) after the visit that holds key j, a bound e_ij on |device logit - exact logit|,
    and the bound e_u(j) on the device's running-max error there (the largest e over the
    keys visited so far: a maximum moves by at most the largest move of its arguments).

    Writing O_i = sum_j c_j e^(m_u(j)) v_j / D_i (c_j the decoded cast code; D_i = S sum_j
    e^(s_ij) for the fp32 row sum, sum_j c_j e^(m_u(j)) for the quantized one), the device's
    O' has every s_ij and m_u moved within those bounds and may round P~·S to any code
    between the codes of the ends of its interval, each end also widened by the relative
    fp32 band FLIP_REL_WINDOW (the device's own exp2 and scaling). With dc_j the largest
    move of the code value, g_j = e^(e_u(j)), G_i = e^(max_j e_ij) and w_j = e^(m_u(j) - m_f):
        dN_ic = sum_j (dc_j g_j + c_j (g_j - 1)) w_j |v_jc|
        fp32:       |O' - O| <= G (dN / L + |O| (G - 1)),       L = S sum_j e^(s_ij - m_f)
        quantized:  |O' - O| <= (dN + |O| dD) / (D - dD),       D = sum_j c_j w_j,
                                                                dD = sum_j (dc_j g_j + c_j (g_j - 1)) w_j
    (|N' - N| <= dN, D'/D within [1/G, G] or D - dD <= D' <= D + dD). With all e = 0 only the
    fp32 band remains. Returns (allow [R, d], flagged [R, N]: more than one admissible code,
    zero_flag [R, N]: admissible codes include zero and a nonzero code, o [R, d])."""
    va = np.abs(np.asarray(v, dtype=np.float64))
    vals, _ = _e4m3_boundaries()
    live = np.isfinite(s)
    e_ij = np.where(live, e_ij, 0.0)
    e_run = np.where(live, e_run, 0.0)
    with np.errstate(invalid="ignore", over="ignore"):
        x = np.where(live, np.exp(s - m_at_key) * S, 0.0)
        m_f = np.where(live, m_at_key, -np.inf).max(axis=1)
        w = np.where(live, np.exp(m_at_key - m_f[:, None]), 0.0)
    spread = e_ij + e_run
    code0 = e4m3.encode(x).astype(np.int64) & 0x7F
    code_lo = e4m3.encode(x * np.exp(-spread) * (1.0 - FLIP_REL_WINDOW)).astype(np.int64) & 0x7F
    # no clip at S: a device's own maximum may come out of its exp2 a rounding above 1
    # (it subtracts a separately rounded product), which matters when S sits on a midpoint
    code_hi = e4m3.encode(np.minimum(x * np.exp(spread) * (1.0 + FLIP_REL_WINDOW), 448.0)).astype(np.int64) & 0x7F
    c0 = np.where(live, vals[code0], 0.0)
    dc = np.where(live, np.maximum(vals[code_hi] - c0, c0 - vals[code_lo]), 0.0)
    flagged = live & (code_lo != code_hi)
    zero_flag = live & (code_lo == 0) & (code_hi != 0)
    g = np.exp(e_run)
    G = np.exp(e_ij.max(axis=1))
    dn_w = (dc * g + c0 * (g - 1.0)) * w
    dN = dn_w @ va
    num = (c0 * w) @ np.asarray(v, dtype=np.float64)
    if denominator == "fp32":
        with np.errstate(invalid="ignore"):
            L = np.where(live, np.exp(s - m_f[:, None]), 0.0).sum(axis=1) * S
        o = num / L[:, None]
        allow = G[:, None] * (dN / L[:, None] + np.abs(o) * (G[:, None] - 1.0))
    elif denominator == "quantized":
        D = (c0 * w).sum(axis=1)
        dD = dn_w.sum(axis=1)
        o = num / D[:, None]
        with np.errstate(divide="ignore"):
            allow = np.where((D > dD)[:, None], (dN + np.abs(o) * dD[:, None]) / (D - dD)[:, None], np.inf)
    else:
        raise ValueError(denominator)
    return allow, flagged, zero_flag, o


def flip_allowance(s, v, *, kv_order: str, S: float, block: int = BLOCK, s_err=None,
                   n_sink: int = N_SINK_DEFAULT, denominator: str = "fp32"):
    """Per-element tolerance of a device output against the oracle on logits ``s``.

    ``s_err`` (optional, [R, N], natural-log units) bounds how far the device's logits may
    lie from ``s`` (see ``mfma_model.logit_error_bound``); without it only the device's own
    fp32 evaluation of P~·S is allowed for: a value within the relative band
    ``FLIP_REL_WINDOW`` of an E4M3 rounding midpoint may be rounded to either neighbour.
    With it, every logit and running max may move within its interval, which widens the set
    of admissible codes and adds the continuous effect on the weights and the row sum (the
    bound is derived in ``_allowance_from``).
    Returns (allow [R, d], flagged [R, N] bool, zero_flagged [R] int: pairs whose admissible
    codes include both zero and a nonzero code, which can move the collapse count).
    """
    s = np.asarray(s, dtype=np.float64)
    m_at_key, _ = _running_max_at_key(s, kv_order, block, n_sink)
    if s_err is None:
        e_ij = np.zeros_like(s)
        e_run = e_ij
    else:
        e_ij = np.where(np.isfinite(s), np.asarray(s_err, dtype=np.float64), 0.0)
        e_run, _ = _running_max_at_key(np.where(np.isfinite(s), e_ij, -np.inf), kv_order, block, n_sink)
        e_run = np.where(np.isfinite(e_run), e_run, 0.0)
    allow, flagged, zero_flag, _ = _allowance_from(s, v, m_at_key, e_ij, e_run, S=S, denominator=denominator)
    return allow, flagged, zero_flag.sum(axis=1)


# --------------------------------------------------------------------------------------
# decode with the key range split (one query row per head)
# --------------------------------------------------------------------------------------

def split_ranges(n_keys: int, n_split: int, block: int = BLOCK):
    """The contiguous key ranges of a split-KV pass: the nb = n_keys / 64 blocks shared as
    evenly as possible, split s holding blocks [floor(s nb / n), floor((s + 1) nb / n))."""
    nb = n_keys // block
    if not 1 <= n_split <= nb:
        raise ValueError("need 1 <= n_split <= number of blocks")
    return [((s * nb // n_split) * block, ((s + 1) * nb // n_split) * block) for s in range(n_split)]


def online_softmax_state(s, v, *, kv_order: str, S: float, p_cast: str = "e4m3", block: int = BLOCK):
    """The recurrence of ``online_softmax_pcast`` over the keys of ``s`` (one split), returned
    unnormalised: (m [R], l [R], acc [R, d]) with l = sum of P~·S and acc = sum P8·v, both
    relative to the final max m of this split."""
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    R, N = s.shape
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, v.shape[1]))
    for (j0, j1) in visit_units(N, kv_order, block, 0):
        sb = s[:, j0:j1]
        live = np.isfinite(sb)
        row_live = live.any(axis=1)
        bmax = np.where(live, sb, -np.inf).max(axis=1)
        m_new = np.where(row_live, np.maximum(m, bmax), m)
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
            p = np.where(live, np.exp(sb - m_new[:, None]), 0.0)
        p8 = _cast(p * S, p_cast)
        l = alpha * l + p.sum(axis=1) * S
        acc = alpha[:, None] * acc + p8 @ v[j0:j1]
        m = m_new
    return m, l, acc


def decode_split(s, v, *, kv_order: str, S: float, n_split: int, p_cast: str = "e4m3", block: int = BLOCK):
    """Split-KV decode: every split runs the online softmax with the P-cast over its own key
    range (its own running max, its blocks in ``kv_order``); the split states are then merged
    exactly: with m = max_s m_s, O = sum_s acc_s e^(m_s - m) / sum_s l_s e^(m_s - m)."""
    parts = [online_softmax_state(s[:, j0:j1], v[j0:j1], kv_order=kv_order, S=S, p_cast=p_cast, block=block)
             for (j0, j1) in split_ranges(s.shape[1], n_split, block)]
    m = np.max(np.stack([p[0] for p in parts]), axis=0)
    num = sum(np.exp(p[0] - m)[:, None] * p[2] for p in parts)
    den = sum(np.exp(p[0] - m) * p[1] for p in parts)
    return num / den[:, None]


def _split_running_max(s, kv_order: str, n_split: int, block: int = BLOCK):
    """Per key, the running max of its own split right after visiting its block (each split
    walks its blocks in ``kv_order`` from -inf), as ``_running_max_at_key`` for one split."""
    out = np.full(s.shape, -np.inf)
    for (j0, j1) in split_ranges(s.shape[1], n_split, block):
        out[:, j0:j1], _ = _running_max_at_key(s[:, j0:j1], kv_order, block, 0)
    return out


def decode_e4m3(q8, k8, v8, q_descale, k_descale, v_descale, *, kv_order: str, S: float, n_split: int,
                logits: str = "exact", with_allowance: bool = False, heads=None,
                qk_accumulation: str = "e4m3_mfma"):
    """Decode oracle over E4M3 inputs: q8 [B, H, d] (one query row per head), k8/v8
    [B, Hkv, N, d]; every query sees all N keys. ``heads``: optional list of (b, h) to
    compute (the others stay 0). Returns dict with ``o`` [B, H, d] and, if asked, ``allow``:
    for exact logits, the tolerance of ``_allowance_from`` with the logit interval of
    ``mfma_model.logit_error_bound`` (``qk_accumulation``) and the split-local running maxima
    (the merged output is sum_j c_j e^(m_u(j)) v_j / (S sum_j e^(s_j)) with m_u(j) the running
    max of key j's own split, so the same bound holds); for device logits, the fp32 band only."""
    B, H, d = q8.shape
    Hkv = k8.shape[1]
    group = H // Hkv
    o = np.zeros((B, H, d))
    allow = np.zeros((B, H, d))
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        hk = h // group
        qrow = q8[b, h][None, :]
        if logits == "exact":
            s, _ = head_logits_e4m3(qrow, k8[b, hk], q_descale[b, h], k_descale[b, hk], d)
        elif logits == "device":
            s = mfma_model.model_logits(qrow, k8[b, hk], q_descale[b, h], k_descale[b, hk], d)
        else:
            raise ValueError(logits)
        vf = e4m3.decode(v8[b, hk]) * float(v_descale[b, hk])
        o[b, h] = decode_split(s, vf, kv_order=kv_order, S=S, n_split=n_split)[0]
        if with_allowance:
            m_at_key = _split_running_max(s, kv_order, n_split)
            if logits == "exact":
                e_ij = mfma_model.logit_error_bound(qrow, k8[b, hk], q_descale[b, h], k_descale[b, hk], d,
                                                    accumulation=qk_accumulation)
                e_run = _split_running_max(e_ij, kv_order, n_split)
            else:
                e_ij = np.zeros_like(s)
                e_run = e_ij
            a, _, _, _ = _allowance_from(s, vf, m_at_key, e_ij, e_run, S=S, denominator="fp32")
            allow[b, h] = a[0]
    res = {"o": o}
    if with_allowance:
        res["allow"] = allow
    return res


# --------------------------------------------------------------------------------------
# whole-tensor driver
# --------------------------------------------------------------------------------------

def attention_e4m3(q8, k8, v8, q_descale, k_descale, v_descale, *, causal: bool, kv_order: str,
                   S: float, rows=None, heads=None, n_sink: int = N_SINK_DEFAULT, logits: str = "exact",
                   with_allowance: bool = False, with_counts: bool = False, denominator: str = "fp32",
                   qk_accumulation: str = "e4m3_mfma"):
    """Oracle over [B, H, N, d] E4M3 inputs (GQA: query head h reads kv head h // (H/Hkv)).

    ``q_descale`` is [B, H], ``k_descale``/``v_descale`` are [B, Hkv]. ``rows`` limits the
    query rows (same subset for every head); ``heads`` is an optional list of (b, h).

    ``logits``: "exact" (the exact dot products of the decoded codes: the pages' result) or
    "device" (the dot products as the gfx950 FP8 matrix core forms them, ``mfma_model``: a
    secondary reference); the rest of the algorithm is identical. ``with_allowance`` adds a
    per-element tolerance (``flip_allowance``):
      * for "exact": the logit interval of ``mfma_model.logit_error_bound`` for the device's
        Q·K^T accumulation ``qk_accumulation`` ("e4m3_mfma": the FP8 matrix core; "fp32": a
        matrix core with exact products and fp32 accumulation), with the fp32 band;
      * for "device": only the fp32 band around its own P~·S.
    Returns dict with ``o`` [len(heads), R, d], ``rows``, ``heads`` and, if asked,
    ``allow`` (same shape as o), ``zero_flagged`` and ``counts`` (summed over heads).
    ``n_sink`` sets the sink tokens of the counts and of "reverse_sink_last";
    ``denominator`` is "fp32" or "quantized" (see ``online_softmax_pcast``).
    """
    if logits not in ("exact", "device"):
        raise ValueError(logits)
    B, H, N, d = q8.shape
    Hkv = k8.shape[1]
    group = H // Hkv
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    outs, allows, zflag = [], [], 0
    counts = np.zeros(4, dtype=np.int64)
    idx = None
    for (b, h) in heads:
        hk = h // group
        if logits == "exact":
            s, idx = head_logits_e4m3(q8[b, h], k8[b, hk], q_descale[b, h], k_descale[b, hk], d,
                                      rows=rows, causal=causal)
        else:
            s = mfma_model.model_logits(q8[b, h], k8[b, hk], q_descale[b, h], k_descale[b, hk], d,
                                        rows=rows, causal=causal)
            idx = np.arange(N) if rows is None else np.asarray(rows)
        vf = e4m3.decode(v8[b, hk]) * float(v_descale[b, hk])
        opts = {"kv_order": kv_order, "S": S, "n_sink": n_sink, "denominator": denominator}
        o, _ = online_softmax_pcast(s, vf, **opts)
        outs.append(o)
        if with_allowance:
            s_err = None
            if logits == "exact":
                s_err = mfma_model.logit_error_bound(q8[b, h], k8[b, hk], q_descale[b, h], k_descale[b, hk], d,
                                                     rows=rows, accumulation=qk_accumulation)
            a, _, z = flip_allowance(s, vf, s_err=s_err, **opts)
            allows.append(a)
            zflag += int(z.sum())
        if with_counts:
            counts += collapse_counts(s, kv_order=kv_order, S=S, n_sink=n_sink)
    res = {"o": np.stack(outs), "rows": idx, "heads": heads}
    if with_allowance:
        res["allow"] = np.stack(allows)
        res["zero_flagged"] = zflag
    if with_counts:
        res["counts"] = counts
    return res
