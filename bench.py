#!/usr/bin/env python3
"""Benchmark of the FP8 (E4M3) P-cast attention forward on one MI355X.

One step = one pass of the whole hot path over the synthetic workload: Q.K^T, the
online softmax in the chosen KV block order, the P.S -> E4M3 cast, P.V, the epilogue,
and the collapse diagnostic, all in the single fused launch of fp8_attn_fwd_counted
(plus the tiny kernel that zeroes the four counters). The default workload is the
long-context GQA causal prefill: B=1, 32 query heads, 8 KV heads, N=32768, d=128,
sink strength 10 on tokens 0..3, reverse order, S=256, per-head E4M3 descale.

Printed: one JSON line with the throughput (TFLOP/s of algorithmic attention FLOP,
4*d per unmasked query-key pair), the roofline of the dominant kernel against the
MI355X dense-FP8 matrix peak, the oracle's CPU throughput on a bounded sample, the
collapse fractions and the output MSE against fp64 attention (with the bf16
FlashAttention comparison).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 attn fwd TFLOP/s (causal, d=128) + %MFMA peak; P-collapse frac & MSE"
PEAK_FP8_TFLOPS = 5000.0          # MI355X dense FP8 matrix peak (no sparsity)
DEFAULT_WORKLOAD = "gqa_causal_h32_kv8_n32768_d128"
KERNEL_SOURCES = ["precision_attention_amd/csrc/fwd.hip", "precision_attention_amd/csrc/fwd16.hip",
                  "precision_attention_amd/csrc/fwd_common.h", "precision_attention_amd/csrc/launch.h",
                  "precision_attention_amd/csrc/kernel_common.h"]
DECODE_SOURCES = ["precision_attention_amd/csrc/decode.hip", "precision_attention_amd/csrc/launch.h",
                  "precision_attention_amd/csrc/kernel_common.h"]


def fused_kernel_name(w) -> str:
    """The fused forward + count kernel this workload launches (S = 256, reverse order)."""
    from precision_attention_amd import binding
    kw = dict(causal=w.causal, kv_order="reverse", S=256.0)
    if binding.fwd_walk_groups(w.B, w.H, w.Hkv, w.N, w.d, **kw) == 2:
        return "fwd_pair_kernel<true, true, true>"
    rows = binding.fwd_tile_rows(w.B, w.H, w.Hkv, w.N, w.d, **kw)
    return "fwd16_kernel<true, true, true>" if rows == 16 else f"fwd_kernel<{w.d}, true, true, true, false, false>"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def strip_comments(text: str) -> str:
    """C++ source without its comments and with whitespace runs collapsed: what the
    compiler sees, so that edits to comments do not change the hash. (The kernel sources
    hold no string or character literals with comment markers.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(sources=None) -> str:
    """Hash of the code (comments stripped) of the sources a kernel is built from (by
    default the prefill kernel's); the measurement records under profiles/ carry the hash
    of the code they were taken on."""
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kind: str = "fwd_counted", n_split=None):
    """HBM bytes per launch (per call, for the decode's two kernels) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel code (and, for the
    decode, at the same split count); else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    sources = DECODE_SOURCES if kind == "decode" else KERNEL_SOURCES
    if rec.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    if n_split is not None and rec.get("n_split") != n_split:
        return None
    return rec.get("hbm_bytes_per_launch")


def quality_heads(H):
    """Heads of batch 0 sampled for the quality figures: 0, 9, 22 and 31 where they exist,
    and the last head."""
    return tuple((0, h) for h in sorted({h for h in (0, 9, 22, 31) if h < H} | {H - 1}))


def quality(inp, w, o_gpu, order, S, n_rows=64, heads=None):
    """MSE of the GPU output against exact fp64 attention on the fp32 source tensors, and
    of a bf16 FlashAttention fed the same E4M3 operands (forward order, P rounded to bf16),
    on sampled rows of ``quality_heads``. Uses the oracle (CPU)."""
    import numpy as np

    heads = quality_heads(w.H) if heads is None else heads

    from oracle import attention as A
    from oracle import e4m3
    from precision_attention_amd import inputs as I

    rows = I.sample_rows(w.N, n_rows, seed=1, edge=8)
    g = w.H // w.Hkv
    se_gpu = se_bf16 = 0.0
    count = 0
    for (b, h) in heads:
        hk = h // g
        s_src, _ = A.head_logits_float(inp["q"][b, h], inp["k"][b, hk], w.d, rows=rows, causal=w.causal)
        ref = A.exact_attention(s_src, inp["v"][b, hk])
        s8, _ = A.head_logits_e4m3(inp["q8"][b, h], inp["k8"][b, hk], inp["qd"][b, h], inp["kd"][b, hk], w.d,
                                   rows=rows, causal=w.causal)
        vf = e4m3.decode(inp["v8"][b, hk]) * float(inp["vd"][b, hk])
        o_bf16, _ = A.online_softmax_pcast(s8, vf, kv_order="forward", S=1.0, p_cast="bf16")
        got = o_gpu[b, h].cpu().numpy()[rows].astype(np.float64)
        se_gpu += float(((got - ref) ** 2).sum())
        se_bf16 += float(((o_bf16 - ref) ** 2).sum())
        count += ref.size
    return {"mse_vs_fp64": se_gpu / count, "bf16_fa_mse_vs_fp64": se_bf16 / count,
            "ratio_to_bf16_fa": se_gpu / se_bf16, "rows_per_head": int(len(rows)), "heads": len(heads),
            "reference": "exact fp64 attention on the fp32 source tensors"}


def cpu_baseline(inp, w, order, S, target_s, chunk=1024):
    """The oracle as it stands (exact logits, block-wise online softmax with the E4M3 cast),
    timed on a bounded sample: query rows of head (0, 0) in a seeded random order, in
    chunks of ``chunk`` rows, until about ``target_s`` seconds have elapsed."""
    import numpy as np

    from oracle import attention as A

    order_rows = np.random.default_rng(3).permutation(w.N)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001 - reporting only
        threads = None
    done, pairs, dt = 0, 0.0, 0.0
    while done < w.N and dt < target_s:
        rows = np.sort(order_rows[done:done + chunk])
        t0 = time.perf_counter()
        A.attention_e4m3(inp["q8"], inp["k8"], inp["v8"], inp["qd"], inp["kd"], inp["vd"], causal=w.causal,
                         kv_order=order, S=S, rows=rows, heads=[(0, 0)])
        dt += time.perf_counter() - t0
        pairs += float((rows + 1).sum()) if w.causal else float(len(rows) * w.N)
        done += len(rows)
    flop = 4.0 * w.d * pairs
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads or 1, "kind": "oracle",
            "sample": f"{done} random query rows of head (0,0) with all their keys, in chunks of {chunk}; "
                      f"exact-logit fp64 oracle, {dt:.1f} s; cores = BLAS threads (elementwise passes use one)",
            "seconds": dt, "host_cpus": len(os.sched_getaffinity(0))}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--order", default="reverse", choices=["reverse", "forward"])
    ap.add_argument("--S", type=float, default=256.0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--construction", default="clean", choices=["clean", "literal"],
                    help="sink construction of the synthetic inputs (clean: the non-sink keys carry no sink "
                         "channel; literal: column 0 of those keys stays random)")
    ap.add_argument("--no-quality", action="store_true", help="skip the CPU MSE check")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the oracle")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the oracle sample")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run --steps device-to-device copies of this many MiB (calibrates HBM counters)")
    args = ap.parse_args()

    if args.copy_mib:
        import torch

        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "steps": args.steps}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the attention of one GPU's "
                                   "share is the whole measured path; multi-GPU runs are not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from precision_attention_amd import binding
    from precision_attention_amd import inputs as I

    w = I.WORKLOADS[args.workload]
    if w.decode:
        return bench_decode(args, w)
    dev = torch.device("cuda:0")
    log(f"bench: generating {w.name} (seed {args.seed})")
    inp = I.make_workload_inputs(w, seed=args.seed, construction=args.construction, keep_float=not args.no_quality)
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev) for k in ("q8", "k8", "v8", "qd", "kd", "vd")}
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
    counts = torch.empty(4, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.fwd_counted(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=w.causal,
                            kv_order=args.order, S=args.S, n_sink=w.n_sink, out=o, counts=counts, stream=stream)

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"bench: timing {args.steps} steps")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_per_step = sum(per) / len(per)
    ms_median = float(np.median(per))
    ms_min = min(per)
    flop = w.flop()
    value = flop / (ms_per_step * 1e-3) / 1e12

    # the forward alone (no counting), for reference
    for _ in range(2):
        binding.fwd(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=w.causal, kv_order=args.order,
                    S=args.S, out=o, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        binding.fwd(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=w.causal, kv_order=args.order,
                    S=args.S, out=o, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    fwd_only_ms = e0.elapsed_time(e1) / args.steps

    # final step's outputs: counts and O for the quality check
    step()
    torch.cuda.synchronize()
    c = counts.cpu().numpy().astype(np.int64)
    collapse = {
        "counts": [int(x) for x in c],
        "presink_fraction": float((c[0] - c[1]) / max(c[2] - c[3], 1)),
        "sink_block_fraction": float(c[1] / max(c[3], 1)),
        "total_fraction": float(c[0] / max(c[2], 1)),
    }

    traffic = measured_traffic(w.name)
    roofline = {"bound": "mfma", "achieved": flop / (ms_per_step * 1e-3) / 1e12, "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": flop / (ms_per_step * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                "traffic": traffic, "kernel": fused_kernel_name(w),
                "flop_per_launch": flop}

    out = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
           "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                      "causal": w.causal, "kv_order": args.order, "S": args.S, "delta": w.delta,
                      "n_sink": w.n_sink, "descale": w.descale, "sink_construction": args.construction, "seed": args.seed},
           "roofline": roofline, "mfma_peak_frac": roofline["frac"], "fwd_only_ms": fwd_only_ms,
           "fwd_only_tflops": flop / (fwd_only_ms * 1e-3) / 1e12, "wall_s_timed": wall,
           "step_ms": {"mean": ms_per_step, "median": ms_median, "min": ms_min},
           "tflops_at_median": flop / (ms_median * 1e-3) / 1e12, "tflops_at_min": flop / (ms_min * 1e-3) / 1e12,
           "collapse": collapse}
    if w.d <= 128:
        # the exact-Q.K^T forward (bf16 matrix cores for Q.K^T, exact products), for reference
        ws = torch.empty(binding.load().fp8_attn_fwd_exact_qk_workspace_bytes(w.B, w.Hkv, w.N, w.d),
                         dtype=torch.uint8, device=dev)

        def step_exact():
            binding.fwd_exact_qk(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], causal=w.causal,
                                 kv_order=args.order, S=args.S, n_sink=w.n_sink, out=o, counts=counts,
                                 workspace=ws, stream=stream)

        for _ in range(2):
            step_exact()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            step_exact()
        e1.record(stream)
        torch.cuda.synchronize()
        ex_ms = e0.elapsed_time(e1) / args.steps
        out["exact_qk_counted_ms"] = ex_ms
        out["exact_qk_counted_tflops"] = flop / (ex_ms * 1e-3) / 1e12
        step()                      # leave the benchmarked step's outputs in o and counts
        torch.cuda.synchronize()

    if not args.no_quality:
        log("bench: quality (MSE vs fp64 on sampled rows, CPU)")
        out["mse"] = quality(inp, w, o, args.order, args.S)
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle on a bounded sample)")
        out["cpu_baseline"] = cpu_baseline(inp, w, args.order, args.S, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def bench_decode(args, w):
    """Split-KV decode (one query row per head over all N keys): HBM-bound, so the roofline
    is the HBM peak against the algorithmic bytes (Q, K, V once, O once)."""
    import numpy as np
    import torch

    from precision_attention_amd import binding
    from precision_attention_amd import inputs as I

    dev = torch.device("cuda:0")
    log(f"bench: generating {w.name} (seed {args.seed})")
    inp = I.make_workload_inputs(w, seed=args.seed, construction=args.construction, keep_float=False)
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev) for k in ("q8", "k8", "v8", "qd", "kd", "vd")}
    n_split = binding.decode_default_splits(w.B, w.Hkv, w.H, w.N)
    o = torch.empty((w.B, w.H, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(binding.load().fp8_attn_decode_workspace_bytes(w.B, w.H, w.d, n_split), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.decode(t["q8"], t["k8"], t["v8"], t["qd"], t["kd"], t["vd"], kv_order=args.order, S=args.S,
                       n_split=n_split, out=o, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = w.bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"metric": "FP8 P-cast split-KV decode, algorithmic GB/s (Q, K, V, O once)", "value": gbs,
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
           "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                      "kv_order": args.order, "S": args.S, "n_split": n_split, "delta": w.delta,
                      "sink_construction": args.construction},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": 8000.0, "unit": "GB/s", "frac": gbs / 8000.0,
                        "traffic": measured_traffic(w.name, "decode", n_split=n_split),
                        "kernel": "decode_kernel<128,pow2> + decode_merge_kernel",
                        "bytes_per_launch": nbytes},
           "tflops": w.flop() / (ms * 1e-3) / 1e12}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
