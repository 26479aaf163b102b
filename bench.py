#!/usr/bin/env python
"""Benchmark of the sparse-MLA decode hot path on one MI355X.

One step = one decode call (split kernel + combine kernel) over one layer's
batch.  The headline workload is B = 80 requests x 64 heads, top-k 512 over a
131072-token context per request, fp8 cache rows, 70/30 recent/older index mix.
`--sets` independent seeded input sets (own Q, indices, page table and rows, in
disjoint regions of one device pool) are cycled so that successive calls gather
cold rows: 16 sets touch ~640 MB, more than the 256 MB Infinity Cache.

Prints ONE JSON line.  Timing uses HIP events on the launch stream.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-MLA decode µs/layer + achieved HBM GB/s (% roofline) at B=1..96"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure


def algorithmic(w, split_only: bool, nsplit: int):
    """(bytes, flops) the method must move / compute for workload w.

    Bytes: valid rows, distinct page-table entries, the top-k list, ctx_len and Q
    are read; out (bf16) and lse (fp32) are written.  When the call is split the
    split kernel does not write out/lse (the combine kernel does).
    """
    i = w.topk_idx.astype(np.int64)
    valid = (i >= 0) & (i < w.ctx_len[:, None])
    n_valid = valid.sum()
    pages = sum(len(np.unique(i[b][valid[b]] // 64)) for b in range(w.B))
    B = w.B
    rd = n_valid * w.row_bytes + 4 * pages + 4 * 512 * B + 4 * B + B * 64 * 576 * 2
    wr = B * 64 * 512 * 2 + B * 64 * 4
    byts = rd + (0 if (split_only and nsplit > 1) else wr)
    flops = n_valid * 64 * (2 * 576 + 2 * 512)
    return int(byts), int(flops)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--sets", type=int, default=16)
    ap.add_argument("--repeats", type=int, default=5)
    ap.add_argument("--nsplit", type=int, default=0, help="force the split count (0 = selector)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        return 2

    import torch
    import sparse_mla_top_amd as smla
    import workloads as W
    from workloads.device import upload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    L = args.sets
    t0 = time.time()
    sets = []
    per_set_pages = None
    pool = None
    for l in range(L):
        w = W.make(3, layer=l, page_base=0 if per_set_pages is None else l * per_set_pages)
        if per_set_pages is None:
            per_set_pages = w.pool_pages
            w = W.make(3, layer=0, page_base=0)
            total = per_set_pages * L * W.PAGE * w.row_bytes
            pool = torch.empty(total, dtype=torch.uint8, device=dev)
        sets.append((w, upload(w, dev, pool=pool)))
    pool_pages = per_set_pages * L
    torch.cuda.synchronize()
    print(f"[bench] generated {L} sets of {sets[0][0].name} in {time.time() - t0:.1f}s "
          f"(pool {pool.numel() / 2**30:.1f} GiB)", file=sys.stderr, flush=True)

    w0 = sets[0][0]
    B = w0.B
    shape = smla.make_shape(B, w0.kv_format, w0.max_pages, pool_pages)
    plan, ws_bytes = smla.plan_for(shape, args.nsplit or None)
    plan_arg = plan
    ws = smla.new_workspace(ws_bytes, dev)
    out = torch.empty((B, 64, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, 64), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def call(k, fn):
        d = sets[k % L][1]
        rc = fn(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, out, lse, shape, plan_arg, ws)
        if rc != 0:
            raise RuntimeError(f"decode failed: {smla.strerror(rc)}")

    def full(*a):
        return smla.decode_raw(*a)

    def split_only(*a):
        return smla.split_raw(*a)

    def timed(fn, steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for k in range(steps):
            fn(k)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / steps     # us per call

    for k in range(args.warmup):
        call(k, full)
    torch.cuda.synchronize()

    full_us = statistics.median(timed(lambda k: call(k, full), args.steps) for _ in range(args.repeats))
    split_us = statistics.median(timed(lambda k: call(k, split_only), args.steps) for _ in range(args.repeats))
    comb_us = None
    if plan.nsplit > 1:
        def comb(k):
            rc = smla.combine_raw(shape, plan_arg, ws, out, lse)
            if rc != 0:
                raise RuntimeError(smla.strerror(rc))
        comb_us = statistics.median(timed(comb, args.steps) for _ in range(args.repeats))

    byts, flops = zip(*(algorithmic(w, True, plan.nsplit) for w, _ in sets))
    split_bytes = float(np.mean(byts))
    split_flops = float(np.mean(flops))
    all_bytes = float(np.mean([algorithmic(w, False, plan.nsplit)[0] for w, _ in sets]))
    achieved = split_bytes / (split_us * 1e-6) / 1e9
    roof_us = max(all_bytes / (HBM_PEAK_GBS * 1e9), split_flops / (BF16_PEAK_TFLOPS * 1e12)) * 1e6

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "split_kernel_b80_traffic.json")
    if os.path.exists(tfile):
        try:
            t = json.load(open(tfile))
            if t.get("plan_nsplit") == plan.nsplit and t.get("kernel_rev") == smla.lib().smla_version():
                traffic = t.get("bytes_per_launch")
        except Exception:
            traffic = None

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        wc = w0
        hp = wc.host_pool()
        n = 0
        tc = time.time()
        while True:
            oracle.decode_workload(wc, pool=hp)
            n += 1
            if time.time() - tc >= args.cpu_seconds:
                break
        cpu_us = (time.time() - tc) / n * 1e6
        cpu = {"value": round(cpu_us, 1), "unit": "us/layer", "cores": oracle.max_threads(), "kind": "oracle",
               "sample": f"fp64 C oracle (OpenMP over request x head) on input set 0 of {wc.name} "
                         f"(B={wc.B}, full batch), {n} calls in {time.time() - tc:.1f}s"}

    res = {
        "metric": METRIC,
        "value": round(full_us, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(full_us / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w0.name, "B": B, "heads": 64, "topk": 512, "ctx_len": int(w0.ctx_len[0]),
            "kv_format": "fp8_e4m3_block128+bf16_rope", "row_bytes": w0.row_bytes,
            "index_mix": "358 of last 8192 tokens + 154 older", "input_sets": L,
            "plan": plan.as_dict(), "split_us": round(split_us, 3),
            "combine_us": None if comb_us is None else round(comb_us, 3),
            "algorithmic_bytes_per_call": int(all_bytes), "algorithmic_flops_per_call": int(split_flops),
            "roofline_us_per_call": round(roof_us, 3),
            "whole_call_frac_of_roofline": round(roof_us / full_us, 4),
            "whole_call_GBps": round(all_bytes / (full_us * 1e-6) / 1e9, 1),
            "mfma_frac": round(split_flops / (split_us * 1e-6) / (BF16_PEAK_TFLOPS * 1e12), 4),
        },
        "roofline": {"kernel": "split_kernel<fp8>", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
