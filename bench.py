#!/usr/bin/env python3
"""Throughput of ring attention's per-device hot path on one MI355X.

Workload (the timed "step"): one rank's share of a 131072-token causal
context sharded zigzag over 8 ranks -- 16384 local queries, 32 query heads
over 8 key/value heads, head_dim 128, bf16 -- run as 8 ring steps, each
against one 16384-token key/value block, the next block copied
device-to-device into a staging slot on a side stream while the current one
computes.  One timed step is one whole ring (ringattn_run, forward with LSE)
over inputs resident in HBM.

Legs reported beside it (same JSON line, `legs`): the same share with every
block resident (all-gather rotation, one fused launch); the HBM-bound merge and
backward preprocess; a matrix-core peak probe; the fp32 512-token ring (all 4
ranks, in microseconds: launch-bound); the 8192-token zigzag ring (all 4
ranks); forward+backward of the 262144-token share and of the 65536 packed
document tokens.  `cpu_baseline`: the fp64 oracle on a bounded sample of the
headline share (and the two small rings in full), on the host's cores.

Throughput is causal-effective: FLOPs = 4 * D * Hq * P for the forward and
10 * D * Hq * P for the backward, P = visible (query, key) pairs; skipped
(masked) work is never counted.

Prints one JSON line.  --gpus N > 1 is refused: this benchmark measures one
GPU's share of the ring.  --summarize-trace turns a rocprofv3 kernel trace of
this script into the markdown tables kept under profiles/.
"""
from __future__ import annotations

import argparse
import contextlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CUs x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
N_CU, BF16_FLOP_PER_CLK_CU = 256, 4096
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_c3_traffic.json")
KERNEL_SOURCES = ("ring_attention_ringattn_amd/csrc/fwd_bf16.hip", "ring_attention_ringattn_amd/csrc/mfma_tile.h",
                  "ring_attention_ringattn_amd/csrc/ra_internal.h",
                  "ring_attention_ringattn_amd/build.py")   # its compiler options shape the kernel too
METRIC = "causal-effective attention TFLOP/s per rank-share (fwd, fwd+bwd); % bf16 MFMA peak"
ALL_LEGS = ("allgather", "hbm", "mfma_peak", "c1", "c2", "c4", "c5")


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


@contextlib.contextmanager
def leg_range(name):
    """A named range around a leg, so a kernel trace taken with markers can be split by leg."""
    import torch
    torch.cuda.nvtx.range_push(f"leg:{name}")
    try:
        yield
    finally:
        torch.cuda.synchronize()
        torch.cuda.nvtx.range_pop()


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


def host_inputs(wname, ranks, with_bwd):
    """Seeded host inputs of a ring: the listed (consecutive) ranks' query rows, every key and value."""
    import numpy as np

    import ring_attention_ringattn_amd as ra
    import synthetic
    w = synthetic.WORKLOADS[wname]
    pos = ra.sharding.shard_positions(w.seq, w.n_shards, w.sharding)
    q_rows = np.concatenate([pos[r] for r in ranks])
    return w, pos, synthetic.make_inputs(w, q_rows=q_rows, backward=with_bwd)


def setup_share(wname, ranks, with_bwd, host=None):
    """Device tensors of a ring: the listed (consecutive) ranks' query shards and all N home blocks."""
    import numpy as np
    import torch

    import ring_attention_ringattn_amd as ra

    w, pos, inp = host if host is not None else host_inputs(wname, ranks, with_bwd)
    n = w.n_shards
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    cv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(dt)
    sl = lambda arr, i: arr[:, :, i * pos[0].size:(i + 1) * pos[0].size]
    s = {
        "w": w, "n": n, "ranks": list(ranks), "pos": pos,
        "q": [cv(sl(inp["q"], i)) for i in range(len(ranks))],
        "k": [cv(inp["k"][:, :, p]) for p in pos],
        "v": [cv(inp["v"][:, :, p]) for p in pos],
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
        s["do"] = [cv(sl(inp["do"], i)) for i in range(len(ranks))]
    shp = s["q"][0].shape
    s["o_acc"] = [torch.empty(shp, dtype=torch.float32, device="cuda") for _ in ranks]
    s["lse"] = [torch.empty(shp[:3], dtype=torch.float32, device="cuda") for _ in ranks]
    s["out"] = [torch.empty(shp, dtype=dt, device="cuda") for _ in ranks]
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


def captured(fn):
    """fn (one ring: its launches on the current stream and the copy stream) captured once as a
    HIP graph; replaying it launches the same kernels without the per-launch host work."""
    import torch
    fn()
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        fn()
    torch.cuda.synchronize()
    return g


def fwd_ring_leg(name, side, steps, warmup, label):
    """Forward ring of every rank of a small workload (all N ranks emulated in one ringattn_run),
    launched eagerly and as a replayed HIP graph of the same ring (these rings are short enough
    for launch latency to matter)."""
    import torch

    import synthetic
    w = synthetic.WORKLOADS[name]
    s = setup_share(name, w.ranks(), with_bwd=False)
    p = sum(s["pairs_per_step"])
    t = timed(lambda: run_fwd(s, side), steps, warmup)
    g = captured(lambda: run_fwd(s, side))
    tg = timed(g.replay, steps, warmup)
    fl = 4.0 * w.head_dim * w.hq * w.batch * p
    del g, s
    torch.cuda.empty_cache()
    return {"workload": label, "visible_pairs_per_head": p, "us_per_ring": round(t * 1e6, 1),
            "fwd_tflops": round(fl / t / 1e12, 3), "pct_peak": round(100.0 * fl / t / 1e12 / PEAK_BF16_TFLOPS, 3),
            "us_per_ring_graph": round(tg * 1e6, 1), "fwd_tflops_graph": round(fl / tg / 1e12, 3)}


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

    # the memory ceiling measured on this GPU, beside the 8 TB/s spec figure: libringattn_tools'
    # nontemporal streaming copy and read-only sweep over 1 GiB, best over a few grid sizes
    import ctypes
    tools = ctypes.CDLL(os.path.join(ROOT, "ring_attention_ringattn_amd", "libringattn_tools.so"))
    tools.ra_tool_hbm_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    tools.ra_tool_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
    nb = 1 << 30
    x = torch.empty(nb // 4, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    sink = torch.empty(8192 * 256, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def call(rc):
        if rc != 0:
            raise RuntimeError(f"libringattn_tools streaming probe failed ({rc})")
    best = {"copy": 0.0, "read": 0.0}
    for blocks in (1024, 2048, 4096, 8192):
        sec = event_time(lambda: call(tools.ra_tool_hbm_copy(x.data_ptr(), y.data_ptr(), nb, blocks, st)), steps, warmup)
        best["copy"] = max(best["copy"], 2 * nb / sec / 1e9)
        sec = event_time(lambda: call(tools.ra_tool_hbm_read(x.data_ptr(), nb, blocks, sink.data_ptr(), st)), steps,
                         warmup)
        best["read"] = max(best["read"], nb / sec / 1e9)
    del x, y, sink
    read_gbs = best["read"]
    res = {"stream_probe": {"bytes": nb, "copy_gbs": round(best["copy"], 1), "read_gbs": round(best["read"], 1),
                            "copy_frac_of_hbm_peak": round(best["copy"] / PEAK_HBM_GBS, 3),
                            "read_frac_of_hbm_peak": round(best["read"] / PEAK_HBM_GBS, 3)}}
    for name, fn, per_row in (("merge", lambda: ra.ringattn_merge(o_a, l_a, o_b, l_b), 3 * (4 * D + 4)),
                              ("bwd_preprocess", lambda: ra.ringattn_bwd_preprocess(out, d_o, delta), 4 * D + 4)):
        sec = event_time(fn, steps, warmup)
        nbytes = B * H * S * per_row
        res[name] = {"us": round(sec * 1e6, 2), "algorithmic_bytes": nbytes,
                     "gbs": round(nbytes / sec / 1e9, 1), "frac_of_hbm_peak": round(nbytes / sec / 1e9 / PEAK_HBM_GBS, 3),
                     "frac_of_stream_read": round(nbytes / sec / 1e9 / read_gbs, 3)}
    return {"workload": "HBM-bound kernels at the 131072-token share's shapes (16384 rows x 32 heads, D = 128): "
                        "standalone LSE merge of two fp32 partials, backward preprocess rowsum(dO * O); a measured "
                        "streaming copy and read of 1 GiB beside them",
            **res}


def event_time(fn, steps, warmup):
    """Seconds per call of fn, from events on torch's current stream (where fn's kernels run)."""
    import torch
    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps / 1e3


class TimingEvents:
    """HIP timing events from libringattn_tools, created without the system-scope memory fence
    an ordinary event performs on completion; read after a device synchronisation."""

    def __init__(self, count):
        import ctypes
        self._ct = ctypes
        self.lib = ctypes.CDLL(os.path.join(ROOT, "ring_attention_ringattn_amd", "libringattn_tools.so"))
        self.lib.ra_tool_event_create.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.ra_tool_event_elapsed_ms.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
        self.lib.ra_tool_event_destroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(count):
            h = ctypes.c_void_p()
            if self.lib.ra_tool_event_create(ctypes.byref(h)) != 0:
                raise RuntimeError("timing event creation failed")
            self.handles.append(h.value)

    def elapsed_ms(self, a, b):
        ms = self._ct.c_float()
        if self.lib.ra_tool_event_elapsed_ms(a, b, self._ct.byref(ms)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for h in self.handles:
            self.lib.ra_tool_event_destroy(h)
        self.handles = []


def mfma_peak_leg(steps, warmup):
    """Measured bf16 matrix-core throughput: back-to-back v_mfma_f32_32x32x16_bf16 on register
    operands over every CU (libringattn_tools' probe kernel), beside the published peak."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "ring_attention_ringattn_amd", "libringattn_tools.so"))
    lib.ra_tool_mfma_peak.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    chains = lib.ra_tool_mfma_chains()
    iters, blocks, threads = 4000, 4 * N_CU, 256
    sink = torch.empty(blocks * threads, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        if lib.ra_tool_mfma_peak(iters, blocks, threads, ctypes.c_void_p(sink.data_ptr()), stream) != 0:
            raise RuntimeError("MFMA probe launch failed")
    sec = event_time(launch, steps, warmup)
    flop = blocks * (threads // 64) * iters * chains * 32 * 32 * 16 * 2
    tf = flop / sec / 1e12
    return {"workload": "matrix-core probe: back-to-back v_mfma_f32_32x32x16_bf16, register operands, "
                        f"{blocks} workgroups of {threads // 64} waves, {iters * chains} products per wave",
            "measured_tflops": round(tf, 1), "spec_tflops": PEAK_BF16_TFLOPS,
            "frac_of_spec": round(tf / PEAK_BF16_TFLOPS, 4),
            "implied_clock_ghz": round(tf * 1e12 / (N_CU * BF16_FLOP_PER_CLK_CU) / 1e9, 3)}


# ------------------------------------------------------------------ CPU baseline (fp64 oracle)

_CPU = {}   # host inputs the forked workers read (set before the pool starts)
CPU_C3_ROWS = 384                        # seeded random rows per query head of the headline sample
CPU_GROUP_ROWS = {"c4": 256, "c5": 512}  # seeded random rows of the forward+backward samples


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    _CPU["limits"] = threadpool_limits(limits=1)   # one BLAS thread per process


def _cpu_task(task):
    """The oracle forward (or forward and backward) of a few query rows of one head against every
    visible key; returns the visible (row, key) pairs."""
    import numpy as np

    import oracle
    wname, h, rows = task
    w, pos_rows, inp = _CPU[wname][:3]
    kvh = h * w.hkv // w.hq
    if wname in ("c4", "c5"):   # GQA group 0 only: query heads 0-3 and kv head 0 were drawn
        doc = _CPU[wname][3]
        mode = "doc_causal" if doc is not None else "causal"
        qd = None if doc is None else doc[pos_rows[rows]]
        oracle.attention_backward(inp["q"][:, h:h + 1, rows], inp["k"], inp["v"], inp["do"][:, h:h + 1, rows],
                                  pos_rows[rows], np.arange(w.seq), mode, qd, doc, row_block=128,
                                  skip_masked_columns=True)
        if doc is None:
            return int((pos_rows[rows] + 1).sum())
        starts = np.concatenate([[0], np.cumsum(np.bincount(doc))])
        return int((pos_rows[rows] - starts[doc[pos_rows[rows]]] + 1).sum())
    oracle.attention_forward(inp["q"][:, h:h + 1, rows], inp["k"][:, kvh:kvh + 1], inp["v"][:, kvh:kvh + 1],
                             pos_rows[rows], np.arange(w.seq), "causal", row_block=128,
                             skip_masked_columns=True)
    return int((pos_rows[rows] + 1).sum())   # visible keys of a causal row at position p: p + 1


def _host_facts():
    import numpy as np
    model = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info()
                                 if p.get("user_api") == "blas"})) or "unknown"
    except Exception:
        blas = "unknown"
    return model, np.__version__, blas


def cpu_baseline(c3_host, budget_s):
    """The fp64 oracle, as it stands, on the host's cores: a fork pool of one-BLAS-thread
    processes over (head, 8 query rows) tasks.  Headline: a bounded sample of the 131072-token
    share (per head CPU_C3_ROWS seeded random rows plus the zigzag chunk edges, all visible keys), for at
    most `budget_s` seconds of wall time; beside it the 512-token fp32 ring and the 8192-token
    ring in full, and forward + backward of bounded samples of the 262144-token share and of the
    packed documents (GQA group 0: query heads 0-3 against kv head 0, per head CPU_GROUP_ROWS seeded
    random rows; at most budget_s / 3 seconds each).  Runs before the GPU is touched (forking then is
    safe)."""
    import multiprocessing

    import numpy as np

    import synthetic
    _CPU.clear()
    wc, _, inpc = c3_host
    rows_pos = np.asarray(inpc["q_rows"])
    _CPU["c3"] = (wc, rows_pos, inpc)
    small = {}
    for name in ("c1", "c2"):
        w, _, inp = host_inputs(name, synthetic.WORKLOADS[name].ranks(), False)
        _CPU[name] = (w, np.asarray(inp["q_rows"]), inp)
        small[name] = w
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    rng = np.random.default_rng(0)
    # GQA group 0 of the 262144-token share (rank 0's rows) and of the packed documents (all rows)
    import ring_attention_ringattn_amd as ra
    group_rows = {}
    for name in ("c4", "c5"):
        w = synthetic.WORKLOADS[name]
        cand = ra.sharding.shard_positions(w.seq, w.n_shards, w.sharding)[0] if name == "c4" else np.arange(w.seq)
        rows = np.sort(rng.choice(cand, CPU_GROUP_ROWS[name], replace=False))
        gq = w.hq // w.hkv
        inp = {"q": synthetic.draw_rows(w, synthetic.TAG_Q, gq, rows, w.value_scale),
               "do": synthetic.draw_rows(w, synthetic.TAG_DO, gq, rows, w.do_scale),
               "k": synthetic.draw_rows(w, synthetic.TAG_K, 1, np.arange(w.seq), w.value_scale),
               "v": synthetic.draw_rows(w, synthetic.TAG_V, 1, np.arange(w.seq), w.value_scale)}
        cu = synthetic.cu_seqlens(w)
        doc = None if cu is None else (np.searchsorted(cu, np.arange(w.seq), side="right") - 1).astype(np.int32)
        _CPU[name] = (w, rows, inp, doc)
        group_rows[name] = gq
    c = wc.seq // (2 * wc.n_shards)
    n_local = rows_pos.size
    tasks = {}
    for h in range(wc.hq):
        rows = np.unique(np.concatenate([rng.choice(n_local, CPU_C3_ROWS, replace=False), [0, c - 1, c, 2 * c - 1]]))
        tasks.setdefault("c3", []).extend(("c3", h, rows[i:i + 8]) for i in range(0, rows.size, 8))
    for name, w in small.items():
        n = _CPU[name][1].size
        tasks[name] = [(name, h, np.arange(i, min(n, i + 64))) for i in range(0, n, 64) for h in range(w.hq)]
    for name, gq in group_rows.items():
        n_rows = CPU_GROUP_ROWS[name]
        tasks[name] = [(name, h, np.arange(i, i + 8)) for i in range(0, n_rows, 8) for h in range(gq)]
    model, npver, blas = _host_facts()
    ctx = multiprocessing.get_context("fork")
    res = {}
    for name in ("c3", "c1", "c2", "c4", "c5"):
        w = _CPU[name][0]
        limit = budget_s if name == "c3" else budget_s / 3 if name in ("c4", "c5") else None
        flop_per_pair = 14.0 if name in ("c4", "c5") else 4.0   # forward + backward: 4 + 10 per D
        # a pool per workload, ended when its budget is spent, so that no task of one workload
        # still runs while the next one is timed
        with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
            done = pairs = 0
            t0 = time.perf_counter()
            for p in pool.imap_unordered(_cpu_task, tasks[name]):
                pairs += p
                done += 1
                if limit is not None and time.perf_counter() - t0 > limit:
                    break
            sec = time.perf_counter() - t0
            pool.terminate()
        res[name] = (done, len(tasks[name]), pairs, sec, flop_per_pair * w.head_dim * pairs / sec / 1e12)
    done, total, pairs, sec, tf = res["c3"]
    return {"value": round(tf, 5), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"fp64 oracle forward (numpy) of {done} of {total} tasks of the 131072-token rank share: "
                      f"per head {CPU_C3_ROWS} seeded random query rows plus the zigzag chunk edges, 8 rows x 1 head per "
                      f"task, all visible keys; {pairs} visible (row, key) pairs over the sampled heads in "
                      f"{sec:.1f} s wall; a fork pool of {workers} processes with one BLAS thread each; "
                      f"host CPU {model}; numpy {npver}; BLAS {blas}",
            "per_config": {
                name: {"workload": label, "tasks": f"{res[name][0]} of {res[name][1]}", "seconds": round(res[name][3], 2),
                       "tflops": round(res[name][4], 5)}
                for name, label in (("c1", "fp32 512-token ring, full forward of all 4 ranks (2 heads, D = 64)"),
                                    ("c2", "8192-token zigzag ring, full forward of all 4 ranks (32/8 heads, "
                                           "D = 128)"),
                                    ("c4", "262144-token share, forward + backward (dQ and the rows' dK, dV "
                                           "contributions) of GQA group 0 (query heads 0-3, kv head 0) on "
                                           f"{CPU_GROUP_ROWS['c4']} seeded random rows of rank 0, all visible keys"),
                                    ("c5", f"packed documents, forward + backward of GQA group 0 on "
                                           f"{CPU_GROUP_ROWS['c5']} seeded random rows of the 65536 tokens, "
                                           "document-causal"))}}


# ------------------------------------------------------------------ trace summaries (profiles/)

def _demangle(name):
    import re
    n = re.sub(r"\(.*", "", name).replace("void ", "")
    return {"_ZN2ra19vt_transpose_kernelILi128EEEvPKDF16bNS_7StridesEiiiPDF16b": "ra::vt_transpose_kernel<128>",
            "_ZN2ra14bwd_pre_kernelILi128EDF16bEEviiiPKT0_S3_NS_7StridesEPf": "ra::bwd_pre_kernel<128, bf16>"}.get(n, n)


def summarize_trace(trace_dir, bench_log):
    """Markdown summary of a rocprofv3 kernel trace of this script.  With a marker trace beside it
    (legs run inside named ranges), launches are grouped by leg; the headline ring's forward step
    launches of the timed rings (the last steps x 8 of that leg) are summarised on their own, with
    the roofline fraction they give."""
    import csv
    import glob
    import re
    line = [l for l in open(bench_log).read().splitlines() if l.startswith("{")][-1]
    bench = json.loads(line)
    kt = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)[0]
    rows = sorted(csv.DictReader(open(kt)), key=lambda r: int(r["Start_Timestamp"]))
    ranges = []
    mk = glob.glob(os.path.join(trace_dir, "**", "*marker_api_trace.csv"), recursive=True)
    if mk:
        for r in csv.DictReader(open(mk[0])):
            msg = r.get("Message") or r.get("Marker_Message") or r.get("Function") or ""
            if msg.startswith("leg:"):
                ranges.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), msg[4:]))

    def leg_of(ts):
        for a, b, n in ranges:
            if a <= ts <= b:
                return n
        return "c3_ring" if ranges else "-"
    agg = {}
    step, step_name = [], None
    for r in rows:
        n = _demangle(r["Kernel_Name"])
        if not (n.startswith("ra::") or n.startswith("__amd_rocclr_copyBuffer")):
            continue
        leg = leg_of(int(r["Start_Timestamp"]))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        agg.setdefault((leg, n, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"])), []).append(dur)
        if leg in ("c3_ring", "-") and n.startswith("ra::fwd_bf16_kernel<128, false"):
            step.append(dur)
            step_name = n
    out = ["| leg | kernel | grid (threads) | block | launches | avg us | min us | max us |",
           "|---|---|---|---|---|---|---|---|"]
    for (leg, n, g, b), d in sorted(agg.items(), key=lambda kv: (kv[0][0], -sum(kv[1]))):
        out.append(f"| {leg} | `{n}` | {g} | {b} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
    k, nsteps = bench["steps"], bench["config"]["ring_steps"]
    timed_steps = step[-k * nsteps:]
    flops = bench["roofline"]["flop_per_launch"]
    tf = sum(flops) * k / (sum(timed_steps) / 1e6) / 1e12 if timed_steps else float("nan")
    per_step = [sum(timed_steps[t::nsteps]) / k for t in range(nsteps)] if timed_steps else []
    head = [
        f"Headline forward step kernel `{step_name}`, the {k} timed rings ({k * nsteps} "
        f"launches, after {bench['warmup']} warm-up rings): average {sum(timed_steps) / len(timed_steps):.1f} us per "
        f"launch; per ring step (us) {[round(x, 1) for x in per_step]}; {tf:.1f} TFLOP/s over the causal-effective "
        f"FLOPs of those launches, frac {tf / PEAK_BF16_TFLOPS:.4f} of {PEAK_BF16_TFLOPS} (the bench line of the same "
        f"run: roofline frac {bench['roofline']['frac']}, {bench['ms_per_step']} ms per ring; 8 x average launch = "
        f"{8 * sum(timed_steps) / len(timed_steps) / 1e3:.3f} ms).", ""]
    return "\n".join(head + out) + "\n\nThe bench line of this run:\n\n    " + line + "\n"


def _counter_rows(path):
    """Per dispatch of a rocprofv3 counter run: (kernel, grid, block, dispatch) -> ({counter: value}, ns)."""
    import csv
    rows, dur = {}, {}
    for r in csv.DictReader(open(path)):
        key = (_demangle(r["Kernel_Name"]), int(r["Grid_Size"]), int(r["Workgroup_Size"]), int(r["Dispatch_Id"]))
        rows.setdefault(key, {})
        rows[key][r["Counter_Name"]] = rows[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        dur[key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return rows, dur


def summarize_counters(run_dirs, cal_dirs, traffic_out=None):
    """Markdown table of the ring library's kernels from rocprofv3 counter runs of this script
    (each run a directory holding *counter_collection.csv; counters of several runs are joined
    per kernel and launch shape).  HBM bytes are FETCH_SIZE and WRITE_SIZE scaled by what the
    same counters read for a plain device copy of known size (`--copy-calibration`, cal_dirs:
    the FETCH_SIZE and the WRITE_SIZE run).  With traffic_out, the forward step kernel's HBM bytes
    per launch are written there for the bench line's roofline."""
    import glob
    find = lambda d: glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
    copy_bytes = 64 * 1024 * 1024 * 4
    cal = {}
    for d in cal_dirs:
        rows, _ = _counter_rows(find(d))
        for (k, g, b, _), c in rows.items():
            if k.startswith("__amd_rocclr_copyBuffer") or "copy" in k.lower():
                for n, v in c.items():
                    cal.setdefault(n, []).append(v)
    # the copies: the largest readings are the 256 MiB copies (the fill before them is smaller)
    fetch_kib = sorted(cal.get("FETCH_SIZE", [0.0]))[-1]
    write_kib = sorted(cal.get("WRITE_SIZE", [0.0]))[-1]
    fscale = copy_bytes / (fetch_kib * 1024) if fetch_kib else float("nan")
    wscale = copy_bytes / (write_kib * 1024) if write_kib else float("nan")
    agg = {}
    for d in run_dirs:
        rows, dur = _counter_rows(find(d))
        for key, c in rows.items():
            k, g, b, _ = key
            if not k.startswith("ra::"):
                continue
            a = agg.setdefault((k, g, b), {"n": {}, "c": {}, "ns": []})
            a["ns"].append(dur[key])
            for n, v in c.items():
                a["c"][n] = a["c"].get(n, 0.0) + v
                a["n"][n] = a["n"].get(n, 0) + 1
    out = ["| kernel | grid (threads) | block | avg us | clock GHz | MFMA busy % | executed TFLOP/s | LDS bank "
           "conflicts | HBM read GB | HBM write GB | HBM TB/s |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    per = {}
    for (k, g, b), a in sorted(agg.items(), key=lambda kv: -sum(kv[1]["ns"])):
        m = {n: a["c"][n] / a["n"][n] for n in a["c"]}
        ns = sum(a["ns"]) / len(a["ns"])
        gui = m.get("GRBM_GUI_ACTIVE")
        clk = gui / 8 / ns if gui else float("nan")
        busy = 100 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui / 8 * 1024) if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in m else float("nan")
        tf = m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", float("nan")) * 512 / ns / 1e3
        rd = m.get("FETCH_SIZE", float("nan")) * 1024 * fscale
        wr = m.get("WRITE_SIZE", float("nan")) * 1024 * wscale
        per[(k, g, b)] = (rd, wr)
        out.append(f"| `{k}` | {g} | {b} | {ns / 1e3:.1f} | {clk:.2f} | {busy:.1f} | {tf:.0f} | "
                   f"{m.get('SQ_LDS_BANK_CONFLICT', float('nan')):.0f} | {rd / 1e9:.3f} | {wr / 1e9:.3f} | "
                   f"{(rd + wr) / ns / 1e3:.2f} |")
    head = (f"Copy calibration: a 256 MiB device copy reads FETCH_SIZE {fetch_kib:.1f} KiB and WRITE_SIZE "
            f"{write_kib:.1f} KiB, so HBM read = FETCH_SIZE x {fscale:.3f}, write = WRITE_SIZE x {wscale:.3f}. "
            "Clock = GRBM_GUI_ACTIVE / 8 XCDs / launch duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
            "(GRBM_GUI_ACTIVE / 8 x 1024 SIMDs); executed TFLOP/s = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / duration "
            "(masked parts of partial tiles included). Averages per launch over the launches of each kernel "
            "and launch shape; durations are those of the counter runs (dispatches serialised).\n\n")
    if traffic_out:
        fwd = [(kgb, v) for kgb, v in per.items() if kgb[0].startswith("ra::fwd_bf16_kernel<128, false")]
        (kgb, (rd, wr)), = [max(fwd, key=lambda x: x[0][1])]
        json.dump({"kernel": kgb[0], "grid_threads": kgb[1],
                   "workload": "131072-token rank share, one ring step (16384 queries x 16384 keys, 32/8 heads, "
                               "D = 128): every launch of the headline ring",
                   "commands": [f"rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_c3_{n} -o run -- "
                                "python3 bench.py --legs \"\" --no-cpu-baseline --steps 1 --warmup 1"
                                for c, n in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write"))]
                               + [f"rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_cal_{n} -o run -- "
                                  "python3 bench.py --copy-calibration"
                                  for c, n in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write"))]
                               + ["python3 bench.py --summarize-counters " + " ".join(run_dirs) + " --calibration "
                                  + " ".join(cal_dirs) + " --traffic-out " + traffic_out],
                   "kernel_source_sha256": kernel_source_hash(),
                   "copy_calibration": {"bytes_read_and_written_per_copy": copy_bytes, "fetch_kib_raw": fetch_kib,
                                        "write_kib_raw": write_kib, "fetch_scale": fscale, "write_scale": wscale},
                   "hbm_fetch_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
                   "hbm_bytes_per_launch": rd + wr,
                   "algorithmic_bytes_per_launch": {"q_bytes": 134217728, "kv_bytes": 67108864,
                                                    "o_acc_read_write": 536870912, "lse_read_write": 4194304},
                   "algorithmic_total": 742391808}, open(traffic_out, "w"), indent=1)
    return head + "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=9, help="timed rings (the Dynamic-CP page's method, section "
                    "'Resultados de benchmarks': 10 runs, first dropped)")
    ap.add_argument("--warmup", type=int, default=6,
                    help="untimed rings first: under sustained load the shader clock settles "
                         "(about 1.5 -> 1.84 GHz on MI355X) within the first ~50 ms")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--legs", default=",".join(ALL_LEGS),
                    help=f"comma-separated legs to run beside the headline ring (of {','.join(ALL_LEGS)}; '' for none)")
    ap.add_argument("--no-bwd", action="store_true", help="skip the forward+backward legs (c4, c5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"),
                    help="print the markdown summary of a rocprofv3 trace of this script and exit (no GPU)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="RUN_DIR",
                    help="print the markdown table of rocprofv3 counter runs of this script and exit (no GPU); "
                         "needs --calibration")
    ap.add_argument("--calibration", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="counter runs of --copy-calibration (FETCH_SIZE, then WRITE_SIZE)")
    ap.add_argument("--traffic-out", help="with --summarize-counters: write the forward step's HBM bytes here")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(*args.summarize_trace), end="")
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.calibration, args.traffic_out), end="")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the ring; --gpus {args.gpus} is not supported "
              "(this build runs on a single MI355X and emulates the ring's ranks on it)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    legs = [x for x in args.legs.split(",") if x]
    if args.no_bwd:
        legs = [x for x in legs if x not in ("c4", "c5")]
    unknown = set(legs) - set(ALL_LEGS)
    if unknown:
        ap.error(f"unknown legs {sorted(unknown)}")

    # host inputs of the headline share, and the CPU baseline, before anything touches the GPU
    host = host_inputs("c3", [args.rank], False)
    cpu = None if args.no_cpu_baseline else cpu_baseline(host, args.cpu_budget)

    import torch
    torch.cuda.set_device(0)
    s = setup_share("c3", [args.rank], with_bwd=False, host=host)
    del host
    side = torch.cuda.Stream()
    n = s["n"]
    w = s["w"]
    flops_step = [4.0 * w.head_dim * w.hq * w.batch * p for p in s["pairs_per_step"]]
    flops_ring = sum(flops_step)

    # Events around every step of every timed ring, recorded on the compute stream inside the
    # timed region: their spans are the step kernel's launch durations.  They are created without
    # the system-scope fence of an ordinary event, which would sit between every two step kernels.
    ev = TimingEvents(2 * n * args.steps)
    handles = [ev.handles[2 * n * i: 2 * n * (i + 1)] for i in range(args.steps)]
    with leg_range("c3_ring"):
        for _ in range(args.warmup):
            run_fwd(s, side)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            run_fwd(s, side, handles[i])
        torch.cuda.synchronize()
        t_ring = (time.perf_counter() - t0) / args.steps
    kern_ms = [sum(ev.elapsed_ms(hs[2 * t], hs[2 * t + 1]) for hs in handles) / args.steps for t in range(n)]
    # each timed ring from its first step's start to its last step's end (the tile tables and step
    # 0's value transpose before the first step are outside this span, inside ms_per_step)
    spans = sorted(ev.elapsed_ms(hs[0], hs[2 * n - 1]) for hs in handles)
    ev.close()
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
        "ring_span_ms": {"min": round(spans[0], 4), "median": round(spans[len(spans) // 2], 4),
                         "mean": round(sum(spans) / len(spans), 4), "max": round(spans[-1], 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                     "kernel": "ra::fwd_bf16_kernel<128,*>",
                     "per_launch_ms": [round(x, 4) for x in kern_ms],
                     "flop_per_launch": flops_step},
        "legs": {},
    }

    if "allgather" in legs:
        with leg_range("allgather"):
            t_ag = timed(lambda: run_fwd_allgather(s), args.steps, args.warmup)
        result["legs"]["fwd_allgather_131072_rank_share"] = {
            "workload": "the same rank share with all 8 K/V blocks resident (all-gather rotation): one fused "
                        "launch over every block, softmax state kept in registers, no ring steps",
            "fwd_ms": round(t_ag * 1e3, 3), "fwd_tflops": round(flops_ring / t_ag / 1e12, 2),
            "pct_peak": round(100.0 * flops_ring / t_ag / 1e12 / PEAK_BF16_TFLOPS, 2)}
    del s
    torch.cuda.empty_cache()
    if "hbm" in legs:
        with leg_range("hbm"):
            result["legs"]["hbm_kernels_131072_rank_share"] = hbm_leg(max(args.steps, 20), args.warmup)
    if "mfma_peak" in legs:
        with leg_range("mfma_peak"):
            result["legs"]["mfma_peak_probe"] = mfma_peak_leg(5, 2)
    if "c1" in legs:
        with leg_range("c1"):
            result["legs"]["fwd_fp32_512_all_ranks"] = fwd_ring_leg(
                "c1", side, max(args.steps, 20), args.warmup,
                "fp32, 2 heads (MHA), D = 64, 512 tokens over 4 contiguous ring shards, causal, all 4 ranks "
                "emulated in one ring (launch-bound: reported in microseconds)")
    if "c2" in legs:
        with leg_range("c2"):
            result["legs"]["fwd_8192_zigzag_all_ranks"] = fwd_ring_leg(
                "c2", side, max(args.steps, 20), args.warmup,
                "bf16, 32/8 heads, D = 128, 8192 tokens over 4 zigzag ring shards of 2048, causal, all 4 ranks "
                "emulated in one ring")
    if "c4" in legs:
        with leg_range("c4"):
            result["legs"]["fwd_bwd_262144_rank_share"] = fwd_bwd_leg(
                "c4", [args.rank], side, args.steps, args.warmup,
                "rank share of a 262144-token causal context over 8 zigzag shards (32768 local queries, "
                "8 steps of 32768-token blocks), 32/8 heads, D=128, bf16, forward + backward")
    if "c5" in legs:
        with leg_range("c5"):
            result["legs"]["fwd_bwd_packed_documents"] = fwd_bwd_leg(
                "c5", [0, 1, 2, 3], side, args.steps, args.warmup,
                "65536 packed tokens of lognormal documents (seed 5: 22 documents), document-causal, "
                "4 contiguous ring shards, all ranks, 32/8 heads, D=128, bf16, forward + backward")

    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
