"""Host logic of bench.py (no GPU): the multi-GPU refusal and the FLOP accounting.

The benchmark's throughput is causal-effective: FLOPs are counted from the number
of visible (query, key) pairs, so that count is checked here against closed forms
of zigzag sharding (every rank sees 2N c^2 + c pairs per head, c = S / 2N) and
against the packed-document count of the seed-5 lognormal stream (each document
of length L contributes L (L + 1) / 2 pairs).
"""
import os
import subprocess

import pytest
import sys

import numpy as np

import bench
import ring_attention_ringattn_amd as ra
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2" in r.stderr and "single MI355X" in r.stderr
    assert r.stdout == ""


def _pairs_per_step(name, rank):
    w = synthetic.WORKLOADS[name]
    pos = ra.sharding.shard_positions(w.seq, w.n_shards, w.sharding)
    return [bench.visible_pairs(pos[rank], pos[ra.sharding.block_of(rank, t, w.n_shards)]) for t in range(w.n_shards)]


def test_zigzag_rank_share_pair_counts():
    for name, total in (("c3", 1_073_750_016), ("c4", 4_294_983_680)):
        w = synthetic.WORKLOADS[name]
        c = w.seq // (2 * w.n_shards)
        steps = _pairs_per_step(name, 0)
        assert sum(steps) == total == 2 * w.n_shards * c * c + c
        # the home block (step 0) adds the diagonal c; every other step sees exactly 2 c^2
        assert steps[0] == 2 * c * c + c and all(p == 2 * c * c for p in steps[1:])
    # every rank of the 8192-token ring sees the same count
    w = synthetic.WORKLOADS["c2"]
    c = w.seq // (2 * w.n_shards)
    assert {sum(_pairs_per_step("c2", r)) for r in range(w.n_shards)} == {2 * w.n_shards * c * c + c}


def test_packed_document_pair_count():
    w = synthetic.WORKLOADS["c5"]
    cu = synthetic.cu_seqlens(w)
    lens = np.diff(cu).astype(np.int64)
    assert len(lens) == 22
    assert int((lens * (lens + 1) // 2).sum()) == 271_551_562
    docs = np.searchsorted(cu, np.arange(w.seq), side="right") - 1
    pos = ra.sharding.shard_positions(w.seq, w.n_shards, w.sharding)
    n = w.n_shards
    total = sum(bench.visible_pairs(pos[r], pos[ra.sharding.block_of(r, t, n)], docs)
                for r in range(n) for t in range(n))
    assert total == 271_551_562


def test_measurement_probes_library_rejects_bad_arguments():
    """libringattn_tools (the benchmark's matrix-core and memory probes) exports its probes and
    rejects bad arguments on the host, before any launch."""
    import ctypes
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "ring_attention_ringattn_amd",
                        "libringattn_tools.so")
    if not os.path.exists(path):
        pytest.skip("libringattn_tools is not built")
    lib = ctypes.CDLL(path)
    lib.ra_tool_mfma_peak.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.ra_tool_hbm_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    lib.ra_tool_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.ra_tool_mfma_chains() == 8
    assert lib.ra_tool_mfma_peak(0, 1, 64, None, None) == -1          # no iterations, no sink
    assert lib.ra_tool_mfma_peak(10, 1, 96, None, None) == -1         # threads not a multiple of 64
    assert lib.ra_tool_hbm_copy(None, None, 16, 1, None) == -1        # null buffers
    assert lib.ra_tool_hbm_copy(16, 32, 15, 1, None) == -1            # size not a multiple of 16
    assert lib.ra_tool_hbm_copy(16, 40, 16, 1, None) == -1            # misaligned destination
    assert lib.ra_tool_hbm_read(16, 16, 0, 64, None) == -1            # no workgroups
    assert lib.ra_tool_hbm_read(None, 16, 1, 64, None) == -1          # null source
    # timing events: null arguments are refused before any runtime call
    lib.ra_tool_event_create.argtypes = [ctypes.c_void_p]
    lib.ra_tool_event_elapsed_ms.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.ra_tool_event_destroy.argtypes = [ctypes.c_void_p]
    assert lib.ra_tool_event_create(None) == -1
    assert lib.ra_tool_event_elapsed_ms(None, None, None) == -1
    assert lib.ra_tool_event_destroy(None) == -1


def test_traffic_counters_are_reported_only_for_the_sources_they_were_taken_on(tmp_path, monkeypatch):
    """roofline.traffic comes from the committed counter summary only while the forward
    kernel's sources (and the build options in build.py) hash to the value recorded with it."""
    import json
    src = tmp_path / "kernel.hip"
    src.write_text("// one version of the kernel\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ("kernel.hip",))
    summary = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(summary))
    assert bench.measured_traffic() is None   # no summary
    summary.write_text(json.dumps({"kernel_source_sha256": bench.kernel_source_hash(), "hbm_bytes_per_launch": 123.0}))
    assert bench.measured_traffic() == 123.0
    src.write_text("// the kernel changed after the counters were taken\n")
    assert bench.measured_traffic() is None


def test_forward_build_options_are_part_of_the_counter_hash():
    assert "ring_attention_ringattn_amd/build.py" in bench.KERNEL_SOURCES
    assert "ring_attention_ringattn_amd/csrc/fwd_bf16.hip" in bench.KERNEL_SOURCES


def test_per_source_compiler_options_reach_only_their_file(monkeypatch, tmp_path):
    from ring_attention_ringattn_amd import build as B
    seen = {}

    class Done:
        returncode, stderr = 0, ""

    def fake_run(cmd, capture_output, text):
        seen[os.path.basename(cmd[cmd.index("-c") + 1])] = cmd
        return Done()
    monkeypatch.setattr(B.subprocess, "run", fake_run)
    for name in ("fwd_bf16.hip", "bwd_bf16.hip"):
        B._compile(os.path.join(B.CSRC, name), (), str(tmp_path))
    assert "--amdgpu-sched-strategy=iterative-ilp" in seen["fwd_bf16.hip"]
    assert not any("sched-strategy" in c for c in seen["bwd_bf16.hip"])
    for cmd in seen.values():   # packed fp32 arithmetic stays off everywhere
        assert "-packed-fp32-ops" in cmd
