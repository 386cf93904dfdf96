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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_c3_traffic.json")
KERNEL_SOURCES = ("ring_attention_ringattn_amd/csrc/fwd_bf16.hip", "ring_attention_ringattn_amd/csrc/mfma_tile.h",
                  "ring_attention_ringattn_amd/csrc/ra_internal.h")


def kernel_source_hash():
    """sha256 over the sources of the forward step kernel (to tell whether counters are stale)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the forward step kernel from the committed counter summary, or None
    when that summary is missing or was taken on other kernel sources."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def copy_calibration():
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 64 * 1024 * 1024
    x = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_copy": n * 4, "bytes_written_per_copy": n * 4,
                      "copies": 3}), flush=True)
METRIC = "causal-effective attention TFLOP/s per rank-share (fwd, fwd+bwd); % bf16 MFMA peak"


def visible_pairs(q_pos, kv_pos, docs=None):
    """Visible (query, key) pairs: keys with kv_pos <= q_pos (and, with documents, in the query's document)."""
    import numpy as np
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    if docs is None:
        ks = np.sort(kv_pos)
        return int(np.searchsorted(ks, q_pos, side="right").sum())
    # documents are contiguous position ranges: count per query the keys in [doc start, q_pos]
    starts = np.zeros(docs.max() + 2, dtype=np.int64)
    starts[1:] = np.cumsum(np.bincount(docs))
    ks = np.sort(kv_pos)
    lo = np.searchsorted(ks, starts[docs[q_pos]], side="left")
    hi = np.searchsorted(ks, q_pos, side="right")
    return int(np.maximum(hi - lo, 0).sum())


def setup_share(wname, ranks, with_bwd):
    """Device tensors of a ring: the listed (consecutive) ranks' query shards and all N home blocks."""
    import numpy as np
    import torch

    import ring_attention_ringattn_amd as ra
    import synthetic

    w = synthetic.WORKLOADS[wname]
    n = w.n_shards
    pos = ra.sharding.shard_positions(w.seq, n, w.sharding)
    q_rows = np.concatenate([pos[r] for r in ranks])
    inp = synthetic.make_inputs(w, q_rows=q_rows, backward=with_bwd)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    sl = lambda arr, i: arr[:, :, i * pos[0].size:(i + 1) * pos[0].size]
    s = {
        "w": w, "n": n, "ranks": list(ranks), "pos": pos, "inp": inp,
        "q": [bf(sl(inp["q"], i)) for i in range(len(ranks))],
        "k": [bf(inp["k"][:, :, p]) for p in pos],
        "v": [bf(inp["v"][:, :, p]) for p in pos],
        "q_pos": [torch.from_numpy(pos[r]).cuda() for r in ranks],
        "kv_pos": [torch.from_numpy(p).cuda() for p in pos],
        "q_doc": None, "kv_doc": None,
        "mask": ra.RA_MASK_DOC_CAUSAL if w.mask == "doc_causal" else ra.RA_MASK_CAUSAL,
    }
    if inp["cu_seqlens"] is not None:
        cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
        s["kv_doc"] = [ra.ringattn_docs_from_cu_seqlens(cu, int(p[0]), p.size) for p in pos]
        s["q_doc"] = [s["kv_doc"][r] for r in ranks]
    if with_bwd:
        s["do"] = [bf(sl(inp["do"], i)) for i in range(len(ranks))]
    shp = s["q"][0].shape
    s["o_acc"] = [torch.empty(shp, dtype=torch.float32, device="cuda") for _ in ranks]
    s["lse"] = [torch.empty(shp[:3], dtype=torch.float32, device="cuda") for _ in ranks]
    s["out"] = [torch.empty(shp, dtype=torch.bfloat16, device="cuda") for _ in ranks]
    docs = None
    if inp["cu_seqlens"] is not None:
        cu_np = inp["cu_seqlens"]
        docs = np.searchsorted(cu_np, np.arange(w.seq), side="right") - 1
    s["pairs_per_step"] = [sum(visible_pairs(pos[r], pos[ra.sharding.block_of(r, t, n)], docs) for r in ranks)
                           for t in range(n)]
    # one workspace for every run mode the legs use: forward ring, all-gather forward, backward ring
    need = [ra.ringattn_run_workspace_size(s["q"][0], s["k"][0], n, len(ranks), pass_=ra.RA_PASS_FWD),
            ra.ringattn_run_workspace_size(s["q"][0], s["k"][0], n, len(ranks), pass_=ra.RA_PASS_FWD,
                                           flags=ra.RA_RUN_ALLGATHER)]
    if with_bwd:
        need.append(ra.ringattn_run_workspace_size(s["q"][0], s["k"][0], n, len(ranks), pass_=ra.RA_PASS_BWD))
    s["ws"] = torch.empty(max(need), dtype=torch.uint8, device="cuda")
    if with_bwd:
        kshp = s["k"][0].shape
        s["delta"] = [torch.empty(shp[:3], dtype=torch.float32, device="cuda") for _ in ranks]
        s["dq"] = [torch.empty(shp, dtype=torch.float32, device="cuda") for _ in ranks]
        s["dk"] = [torch.empty(kshp, dtype=torch.float32, device="cuda") for _ in range(n)]
        s["dv"] = [torch.empty(kshp, dtype=torch.float32, device="cuda") for _ in range(n)]
    return s


def run_fwd(s, side, events=None):
    import ring_attention_ringattn_amd as ra
    ra.ringattn_run(s["q"], s["k"], s["v"], s["q_pos"], s["kv_pos"], o_acc=s["o_acc"], lse=s["lse"], out=s["out"],
                    q_doc=s["q_doc"], kv_doc=s["kv_doc"], first_rank=s["ranks"][0], mask_mode=s["mask"],
                    workspace=s["ws"], copy_stream=side, step_events=events)


def run_fwd_allgather(s):
    """The same share with every block resident: one fused launch over all N blocks (no ring)."""
    import ring_attention_ringattn_amd as ra
    ra.ringattn_run(s["q"], s["k"], s["v"], s["q_pos"], s["kv_pos"], lse=s["lse"], out=s["out"],
                    q_doc=s["q_doc"], kv_doc=s["kv_doc"], first_rank=s["ranks"][0], mask_mode=s["mask"],
                    workspace=s["ws"], flags=ra.RA_RUN_ALLGATHER)


def run_bwd(s, side):
    import ring_attention_ringattn_amd as ra
    for t in s["dq"] + s["dk"] + s["dv"]:
        t.zero_()
    ra.ringattn_run(s["q"], s["k"], s["v"], s["q_pos"], s["kv_pos"], lse=s["lse"], out=s["out"], d_o=s["do"],
                    q_doc=s["q_doc"], kv_doc=s["kv_doc"], delta=s["delta"], dq=s["dq"], dk=s["dk"], dv=s["dv"],
                    first_rank=s["ranks"][0], mask_mode=s["mask"], pass_=ra.RA_PASS_BWD, workspace=s["ws"],
                    copy_stream=side)


def fwd_bwd_leg(name, ranks, side, steps, warmup, label):
    import torch
    s = setup_share(name, ranks, with_bwd=True)
    w = s["w"]
    p = sum(s["pairs_per_step"])
    t_f = timed(lambda: run_fwd(s, side), steps, warmup)
    t_b = timed(lambda: run_bwd(s, side), steps, warmup)
    fl_f, fl_b = 4.0 * w.head_dim * w.hq * w.batch * p, 10.0 * w.head_dim * w.hq * w.batch * p
    del s
    torch.cuda.empty_cache()
    return {"workload": label, "visible_pairs_per_head": p,
            "fwd_ms": round(t_f * 1e3, 3), "bwd_ms": round(t_b * 1e3, 3),
            "fwd_tflops": round(fl_f / t_f / 1e12, 2), "bwd_tflops": round(fl_b / t_b / 1e12, 2),
            "fwd_bwd_tflops": round((fl_f + fl_b) / (t_f + t_b) / 1e12, 2),
            "fwd_bwd_pct_peak": round(100.0 * (fl_f + fl_b) / (t_f + t_b) / 1e12 / PEAK_BF16_TFLOPS, 2)}


def hbm_leg(steps, warmup):
    """The HBM-bound kernels at the 131072-token share's shapes (16384 rows x 32 heads, D = 128):
    the standalone LSE merge of two fp32 partials, (o_b, lse_b) <- (o_a, lse_a) (+) (o_b, lse_b),
    which reads 2 (4D + 4) and writes 4D + 4 bytes per row and head (1548 B), and the backward
    preprocess delta = rowsum(dO * O) over bf16 O and dO, 4D + 4 bytes per row and head (516 B).
    Timed with events on the stream the kernels run on (torch's current stream)."""
    import torch

    import ring_attention_ringattn_amd as ra
    B, H, S, D = 1, 32, 16384, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    o_a, o_b = (torch.randn(B, H, S, D, device="cuda", generator=g) for _ in range(2))
    l_a, l_b = (torch.randn(B, H, S, device="cuda", generator=g) for _ in range(2))
    out, d_o = (torch.randn(B, H, S, D, device="cuda", generator=g).to(torch.bfloat16) for _ in range(2))
    delta = torch.empty(B, H, S, device="cuda")

    def t(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps / 1e3

    res = {}
    for name, fn, per_row in (("merge", lambda: ra.ringattn_merge(o_a, l_a, o_b, l_b), 3 * (4 * D + 4)),
                              ("bwd_preprocess", lambda: ra.ringattn_bwd_preprocess(out, d_o, delta), 4 * D + 4)):
        sec = t(fn)
        nbytes = B * H * S * per_row
        res[name] = {"us": round(sec * 1e6, 2), "algorithmic_bytes": nbytes,
                     "gbs": round(nbytes / sec / 1e9, 1), "frac_of_hbm_peak": round(nbytes / sec / 1e9 / PEAK_HBM_GBS, 3)}
    return {"workload": "HBM-bound kernels at the 131072-token share's shapes (16384 rows x 32 heads, D = 128): "
                        "standalone LSE merge of two fp32 partials, backward preprocess rowsum(dO * O)",
            **res}


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
    ap.add_argument("--warmup", type=int, default=6,
                    help="untimed rings first: under sustained load the shader clock settles "
                         "(about 1.5 -> 1.84 GHz on MI355X) within the first ~50 ms")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--no-bwd", action="store_true", help="skip the forward+backward legs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the ring; --gpus {args.gpus} is not supported "
              "(this build runs on a single MI355X and emulates the ring's ranks on it)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import ring_attention_ringattn_amd as ra

    torch.cuda.set_device(0)
    s = setup_share("c3", [args.rank], with_bwd=False)
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
        # ring time not covered by the step kernels: launch gaps between steps, the tile tables, the
        # transpose of step 0's home value block on the compute stream, and any wait for a staging copy
        "exposed_ms_per_ring": round(t_ring * 1e3 - sum(kern_ms), 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                     "kernel": "ra::fwd_bf16_kernel<128,*>",
                     "per_launch_ms": [round(x, 4) for x in kern_ms],
                     "flop_per_launch": flops_step},
    }

    # the all-gather rotation on the same share: every block resident, one fused launch
    t_ag = timed(lambda: run_fwd_allgather(s), args.steps, args.warmup)
    result["legs"] = {"fwd_allgather_131072_rank_share": {
        "workload": "the same rank share with all 8 K/V blocks resident (all-gather rotation): one fused "
                    "launch over every block, softmax state kept in registers, no ring steps",
        "fwd_ms": round(t_ag * 1e3, 3), "fwd_tflops": round(flops_ring / t_ag / 1e12, 2),
        "pct_peak": round(100.0 * flops_ring / t_ag / 1e12 / PEAK_BF16_TFLOPS, 2)}}

    result["legs"]["hbm_kernels_131072_rank_share"] = hbm_leg(max(args.steps, 20), args.warmup)

    if not args.no_bwd:
        del s
        torch.cuda.empty_cache()
        result["legs"].update({
            "fwd_bwd_262144_rank_share": fwd_bwd_leg(
                "c4", [args.rank], side, args.steps, args.warmup,
                "rank share of a 262144-token causal context over 8 zigzag shards (32768 local queries, "
                "8 steps of 32768-token blocks), 32/8 heads, D=128, bf16, forward + backward"),
            "fwd_bwd_packed_documents": fwd_bwd_leg(
                "c5", [0, 1, 2, 3], side, args.steps, args.warmup,
                "65536 packed tokens of lognormal documents (seed 5: 22 documents), document-causal, "
                "4 contiguous ring shards, all ranks, 32/8 heads, D=128, bf16, forward + backward"),
        })

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(*host, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
