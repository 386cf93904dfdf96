#!/usr/bin/env python3
"""Throughput of ring attention's per-device hot path on one MI355X.

Workload (default): one rank's share of a 131072-token causal context sharded
zigzag over 8 ranks -- 16384 local queries, 32 query heads over 8 key/value
heads, head_dim 128, bf16 -- run as 8 ring steps, each against one
16384-token key/value block, the next block copied device-to-device into a
staging slot on a side stream while the current one computes.  One timed
"step" is one whole ring (ringattn_run, forward with LSE) over resident
inputs.  Optionally (--bwd) a second leg times forward+backward of the
262144-token share (32768 local queries, 8 blocks of 32768 keys).

Throughput is causal-effective: FLOPs = 4 * D * Hq * P for the forward and
10 * D * Hq * P for the backward, P = visible (query, key) pairs; skipped
(masked) work is never counted.

Prints one JSON line.  --gpus N > 1 is refused: this benchmark measures one
GPU's share of the ring.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CUs x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
METRIC = "causal-effective attention TFLOP/s per rank-share (fwd, fwd+bwd); % bf16 MFMA peak"


def visible_pairs(q_pos, kv_pos):
    """Causal visible (query, key) pairs: sum over queries of keys with kv_pos <= q_pos."""
    import numpy as np
    ks = np.sort(np.asarray(kv_pos, dtype=np.int64))
    return int(np.searchsorted(ks, np.asarray(q_pos, dtype=np.int64), side="right").sum())


def setup_share(wname, rank, with_bwd):
    import numpy as np
    import torch

    import ring_attention_ringattn_amd as ra
    import synthetic

    w = synthetic.WORKLOADS[wname]
    n = w.n_shards
    pos = ra.sharding.shard_positions(w.seq, n, w.sharding)
    inp = synthetic.make_inputs(w, q_rows=pos[rank], backward=with_bwd)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    s = {
        "w": w, "n": n, "rank": rank, "pos": pos, "inp": inp,
        "q": [bf(inp["q"])],
        "k": [bf(inp["k"][:, :, p]) for p in pos],
        "v": [bf(inp["v"][:, :, p]) for p in pos],
        "q_pos": [torch.from_numpy(pos[rank]).cuda()],
        "kv_pos": [torch.from_numpy(p).cuda() for p in pos],
    }
    if with_bwd:
        s["do"] = [bf(inp["do"])]
    shp = s["q"][0].shape
    s["o_acc"] = [torch.empty(shp, dtype=torch.float32, device="cuda")]
    s["lse"] = [torch.empty(shp[:3], dtype=torch.float32, device="cuda")]
    s["out"] = [torch.empty(shp, dtype=torch.bfloat16, device="cuda")]
    s["pairs_per_step"] = [visible_pairs(pos[rank], pos[ra.sharding.block_of(rank, t, n)]) for t in range(n)]
    s["ws"] = torch.empty(ra.ringattn_run_workspace_size(s["q"][0], s["k"][0], n, 1), dtype=torch.uint8,
                          device="cuda")
    return s


def run_fwd(s, side, events=None):
    import ring_attention_ringattn_amd as ra
    ra.ringattn_run(s["q"], s["k"], s["v"], s["q_pos"], s["kv_pos"], o_acc=s["o_acc"], lse=s["lse"], out=s["out"],
                    first_rank=s["rank"], workspace=s["ws"], copy_stream=side, step_events=events)


def run_bwd(s, side):
    import ring_attention_ringattn_amd as ra
    for t in s["dq"] + s["dk"] + s["dv"]:
        t.zero_()
    ra.ringattn_run(s["q"], s["k"], s["v"], s["q_pos"], s["kv_pos"], lse=s["lse"], out=s["out"], d_o=s["do"],
                    delta=s["delta"], dq=s["dq"], dk=s["dk"], dv=s["dv"], first_rank=s["rank"],
                    pass_=ra.RA_PASS_BWD, workspace=s["ws"], copy_stream=side)


def timed(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def cpu_baseline(w, inp, pos, budget_s):
    """The fp64 oracle on a bounded sample of the same share: evenly spread query rows, all 32 heads."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    kpos = np.arange(w.seq)
    done_rows, done_pairs, spent = 0, 0, 0.0
    n_rows = 4
    rng = np.random.default_rng(0)
    while spent < budget_s and done_rows < pos.size:
        idx = np.sort(rng.choice(pos.size, n_rows, replace=False))
        t0 = time.perf_counter()
        oracle.attention_forward(inp["q"][:, :, idx], inp["k"], inp["v"], pos[idx], kpos, "causal",
                                 row_block=128, skip_masked_columns=True)
        spent += time.perf_counter() - t0
        done_rows += n_rows
        done_pairs += visible_pairs(pos[idx], kpos)
        n_rows = min(64, n_rows * 2)
    flops = 4.0 * w.head_dim * w.hq * w.batch * done_pairs
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle forward of {done_rows} query rows of the same rank share (all {w.hq} heads, "
                      f"all visible keys of the 131072-token context), {spent:.1f} s, "
                      f"{done_pairs} visible pairs per head; host {platform.processor() or platform.machine()}, "
                      f"{len(os.sched_getaffinity(0))} cores available"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=9, help="timed rings (the pages' method: 10 runs, first dropped)")
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--bwd", action="store_true", help="also time forward+backward of the 262144-token share")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the ring; --gpus {args.gpus} is not supported "
              "(this build runs on a single MI355X and emulates the ring's ranks on it)", file=sys.stderr)
        sys.exit(2)

    import torch
    import ring_attention_ringattn_amd as ra

    torch.cuda.set_device(0)
    s = setup_share("c3", args.rank, with_bwd=False)
    side = torch.cuda.Stream()
    n = s["n"]
    w = s["w"]
    flops_step = [4.0 * w.head_dim * w.hq * w.batch * p for p in s["pairs_per_step"]]
    flops_ring = sum(flops_step)

    host = (w, s["inp"], s["pos"][args.rank])   # kept for the CPU baseline
    # Events around every step of every timed ring, recorded on the compute stream inside the
    # timed region: their spans are the step kernel's launch durations.
    ev_sets = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * n)] for _ in range(args.steps)]
    for es in ev_sets:
        for e in es:
            e.record()        # creates the underlying hipEvent_t
    handles = [[e.cuda_event for e in es] for es in ev_sets]
    for _ in range(args.warmup):
        run_fwd(s, side)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_fwd(s, side, handles[i])
    torch.cuda.synchronize()
    t_ring = (time.perf_counter() - t0) / args.steps
    kern_ms = [sum(es[2 * t].elapsed_time(es[2 * t + 1]) for es in ev_sets) / args.steps for t in range(n)]
    achieved = flops_ring / (sum(kern_ms) / 1e3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(flops_ring / t_ring / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_ring * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*0.5 bf16 inputs; no dataset or weights)",
        "config": {"workload": "rank share of a 131072-token causal context over 8 zigzag ring shards: "
                               "16384 local queries, 8 ring steps of 16384-token K/V blocks, 32/8 GQA heads, "
                               "head_dim 128, bf16, forward with LSE, K/V prefetch double-buffered on a side stream",
                   "rank": args.rank, "global_batch": 1, "seq_len": w.seq, "local_queries": int(s["pos"][args.rank].size),
                   "ring_steps": n, "parallelism": "cp8 (ring emulated on one GPU)"},
        "pct_peak": round(100.0 * flops_ring / t_ring / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "ra::fwd_bf16_kernel<128,*>",
                     "per_launch_ms": [round(x, 4) for x in kern_ms],
                     "flop_per_launch": flops_step},
    }

    if args.bwd:
        del s
        torch.cuda.empty_cache()
        b = setup_share("c4", args.rank, with_bwd=True)
        shp, kshp = b["q"][0].shape, b["k"][0].shape
        b["delta"] = [torch.empty(shp[:3], dtype=torch.float32, device="cuda")]
        b["dq"] = [torch.empty(shp, dtype=torch.float32, device="cuda")]
        b["dk"] = [torch.empty(kshp, dtype=torch.float32, device="cuda") for _ in range(b["n"])]
        b["dv"] = [torch.empty(kshp, dtype=torch.float32, device="cuda") for _ in range(b["n"])]
        b["ws"] = torch.empty(ra.ringattn_run_workspace_size(b["q"][0], b["k"][0], b["n"], 1, pass_=ra.RA_PASS_BWD),
                              dtype=torch.uint8, device="cuda")
        p = sum(b["pairs_per_step"])
        wb = b["w"]
        t_f = timed(lambda: run_fwd(b, side), args.steps, args.warmup)
        t_b = timed(lambda: run_bwd(b, side), args.steps, args.warmup)
        fl_f, fl_b = 4.0 * wb.head_dim * wb.hq * p, 10.0 * wb.head_dim * wb.hq * p
        result["fwd_bwd"] = {"workload": "rank share of a 262144-token causal context over 8 zigzag shards "
                                         "(32768 local queries, 8 steps of 32768-token blocks), bf16",
                             "fwd_ms": round(t_f * 1e3, 3), "bwd_ms": round(t_b * 1e3, 3),
                             "fwd_tflops": round(fl_f / t_f / 1e12, 2), "bwd_tflops": round(fl_b / t_b / 1e12, 2),
                             "fwd_bwd_tflops": round((fl_f + fl_b) / (t_f + t_b) / 1e12, 2)}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(*host, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
