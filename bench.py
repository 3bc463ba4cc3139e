"""Benchmark of split-KV verify attention on one MI355X.

Workload: 1 sequence, B=16 drafted rows, 24 query heads over 4 KV heads,
head_dim 256, 8-bit KV (int8 + fp16 scale per 32 dims), 32,768-token context,
bf16 Q, fp16 output, synthetic seeded data.  A step is one verify_attn_run
(partial kernel + log-sum-exp merge) with Q, KV, block table and workspace
already resident in HBM.  Eight distinct KV pools (8 x 71 MB, well beyond the
256 MB Infinity Cache) are rotated so every step streams cold KV.

Prints one JSON line.  value = KV bytes of the valid tokens / time per call
(GB/s); roofline = the partial kernel's algorithmic KV bytes / its average
duration (HIP events on the launch stream) against the 8 TB/s HBM peak;
cpu_baseline = the fp64 oracle timed on the host cores for one full call.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify-attn µs/call + achieved HBM GB/s, B=16 H24/KV4/D256 Q8 KV ctx 32K"
HBM_PEAK_GBPS = 8000.0
NPOOLS = 8


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ctx", type=int, default=32768)
    ap.add_argument("--splits", type=int, default=0, help="0 = the plan's heuristic")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--pools", type=int, default=NPOOLS)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import speculative_decoding_verify_kv_amd as va
    import synthetic as S
    from speculative_decoding_verify_kv_amd import device as vdev

    if not os.path.exists(va.LIB_PATH):
        from speculative_decoding_verify_kv_amd import build as vbuild

        vbuild.build()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    t0 = time.time()
    w = S.q8_long(ctx=args.ctx)
    print(f"[bench] generated {w.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = vdev.to_device(w)
    # distinct pools: page-rolled device copies (same values, different memory)
    pools = []
    for r in range(args.pools):
        if r == 0:
            pools.append((dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"]))
        else:
            pools.append(tuple(torch.roll(t, shifts=r * 7, dims=0).contiguous() for t in pools[0]))
    # the rolled pools hold page p at p + 7r: shift the block table accordingly
    tables = [torch.remainder(dev["block_table"] + r * 7, w.num_pages).to(torch.int32).contiguous()
              for r in range(args.pools)]
    prob = vdev.problem_for(w, out_dtype="f16")
    plan = va.verify_attn_plan(prob, args.splits, 0)
    info = plan.info()
    ws = vdev.workspace(plan)
    out, lse = vdev.empty_out(w, "f16")
    kv_bytes = w.kv_bytes_valid()

    def step(i, which="run"):
        k, v, ks, vs = pools[i % args.pools]
        fn = {"run": va.verify_attn_run, "partial": va.verify_attn_run_partial}[which]
        fn(plan, dev["q"], k, v, ks, vs, tables[i % args.pools], dev["ctx_lens"], None, 0, out, lse, ws,
           stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` whole calls ----
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    gbps = kv_bytes / (ms_per_step * 1e-3) / 1e9

    # ---- per-kernel durations on the launch stream (same steps, events between launches) ----
    S_used = info.num_splits
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        a, b, c = evs[i]
        a.record(stream)
        step(i, "partial")
        b.record(stream)
        if S_used > 1:
            va.verify_attn_run_merge(plan, 0, out, lse, ws, stream=stream)
        c.record(stream)
    torch.cuda.synchronize()
    partial_ms = [a.elapsed_time(b) for a, b, _ in evs]
    merge_ms = [b.elapsed_time(c) for _, b, c in evs]
    partial_avg_us = 1e3 * sum(partial_ms) / len(partial_ms)
    merge_avg_us = 1e3 * sum(merge_ms) / len(merge_ms)
    achieved = kv_bytes / (partial_avg_us * 1e-6) / 1e9
    flags = va.verify_attn_read_flags(plan, ws, stream)

    # ---- CPU baseline: the fp64 oracle on the host cores, one full call ----
    cpu = None
    if not args.no_cpu:
        import oracle

        nthreads = oracle.default_threads()
        t0 = time.perf_counter()
        oracle.attention(w, nthreads=nthreads)
        dt = time.perf_counter() - t0
        cpu = {"value": kv_bytes / dt / 1e9, "unit": "GB/s", "cores": nthreads, "kind": "oracle",
               "sample": f"one full call of the same workload (all {w.num_seqs * w.B * w.H} row-heads, "
                         f"ctx {args.ctx}), {dt:.2f} s wall on {nthreads} threads",
               "seconds_per_call": dt}

    rec = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "us_per_call": ms_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": 1, "B": 16, "H": 24, "KVH": 4, "D": 256, "ctx": args.ctx,
                   "kv": "q8_0", "q": "bf16", "out": "f16", "splits": S_used, "row_groups": info.row_groups,
                   "kv_pools_rotated": args.pools, "kv_bytes_per_call": kv_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "verify_partial_kernel<256,Q8,3>", "kernel_avg_us": round(partial_avg_us, 3),
                     "merge_avg_us": round(merge_avg_us, 3)},
        "cpu_baseline": cpu,
        "flags": flags,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
