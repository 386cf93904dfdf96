"""Seeded input generator reproducibility and the fixed facts the pages print."""
import json
import os

import numpy as np

import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_attention_matrix_memory_fact():
    g = json.load(open(os.path.join(GOLDEN, "attention_matrix_memory.json")))
    s = g["seq_len"]
    assert s * s * g["bytes_per_element_bf16"] == g["bytes_per_head"] == 2 ** 35
    assert g["bytes_per_head"] / 2 ** 30 == g["gib_per_head"]
    # the Accelerate guide's "~32 GB" (section "Por que paralelismo de contexto?") also holds
    # for the decimal reading 128000
    assert abs(128000 ** 2 * 2 / 1e9 - 32.768) < 1e-9


def test_packed_document_lengths_seed5():
    lens = synthetic.doc_lengths(5, 65536)
    assert len(lens) == 22 and sum(lens) == 65536
    assert min(lens) == 256 and max(lens) == 14565
    assert sum(n * (n + 1) // 2 for n in lens) == 271_551_562
    cu = synthetic.cu_seqlens(synthetic.WORKLOADS["c5"])
    assert cu.dtype == np.int32 and cu[0] == 0 and cu[-1] == 65536 and cu.size == 23


def test_bf16_round_is_rne():
    # bf16 keeps 7 fraction bits: one ulp at 1.0 is 2**-7
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 2 ** -7 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5e-3], dtype=np.float32)
    r = synthetic.bf16_round(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                        # half an ulp above an even value: stays
    assert r[2] == np.float32(1.0 + 2 ** -6)  # half an ulp above an odd value: goes to the even one
    assert r[3] == np.float32(1.0 + 2 ** -7)  # three quarters of an ulp: rounds up
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)


def test_rows_are_reproducible_and_sliceable():
    w = synthetic.small_workload("c2", seq=1024, n_shards=4)
    full = synthetic.draw_rows(w, synthetic.TAG_Q, 2, np.arange(1024), 0.5)
    rows = np.array([5, 900, 128, 127, 1023])
    part = synthetic.draw_rows(w, synthetic.TAG_Q, 2, rows, 0.5)
    assert np.array_equal(part, full[:, :, rows])
    again = synthetic.draw_rows(w, synthetic.TAG_Q, 2, np.arange(1024), 0.5)
    assert np.array_equal(full, again)
    assert abs(full.std() - 0.5) < 0.02
    assert np.all((full.view(np.uint32) & 0xFFFF) == 0)     # bf16-exact values
