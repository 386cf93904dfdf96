"""Helpers of the GPU parity tests: device tensors from the seeded inputs, runs
through the C ABI (via the binding), and comparisons with the fp64 oracle.

Inputs come from ``synthetic``; expected values only from ``oracle``.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import ring_attention_ringattn_amd as ra
import synthetic

MASKS = {"none": ra.RA_MASK_NONE, "causal": ra.RA_MASK_CAUSAL, "doc_causal": ra.RA_MASK_DOC_CAUSAL}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(x, dtype=torch.float32):
    """Device tensor holding exactly the values of a numpy array (bf16 inputs are bf16-exact)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype)


def thd_view(x_bhsd: torch.Tensor) -> torch.Tensor:
    """Store a [1, H, S, D] tensor token-major ([S, H, D]) and return the [1, H, S, D] view of it."""
    assert x_bhsd.shape[0] == 1
    thd = x_bhsd[0].permute(1, 0, 2).contiguous()
    return thd.permute(1, 0, 2).unsqueeze(0)


def print_case(msg):
    print(f"[case] {msg}", flush=True)


class Ring:
    """One ring on the device: R emulated ranks (first_rank..), N home blocks."""

    def __init__(self, q_glob, k_glob, v_glob, pos_per_rank, mask, dtype, ranks, doc=None, layout="bhsd",
                 do_glob=None, q_shards=None, do_shards=None):
        """q_glob/do_glob: global [B,H,S,D] arrays, or None with q_shards/do_shards given per emulated rank."""
        self.n = len(pos_per_rank)
        self.ranks = list(ranks)
        assert all((self.ranks[0] + i) % self.n == r for i, r in enumerate(self.ranks))
        self.mask = mask
        self.dt = TORCH_DT[dtype]
        self.pos = pos_per_rank
        self.doc = doc
        mk = (lambda a: thd_view(dev(a, self.dt))) if layout == "thd" else (lambda a: dev(a, self.dt))
        if q_shards is None:
            q_shards = [q_glob[:, :, pos_per_rank[r]] for r in self.ranks]
        if do_shards is None and do_glob is not None:
            do_shards = [do_glob[:, :, pos_per_rank[r]] for r in self.ranks]
        self.q = [mk(x) for x in q_shards]
        self.k = [mk(k_glob[:, :, p]) for p in pos_per_rank]
        self.v = [mk(v_glob[:, :, p]) for p in pos_per_rank]
        self.do = None if do_shards is None else [mk(x) for x in do_shards]
        self.q_pos = [dev(pos_per_rank[r], torch.int32) for r in self.ranks]
        self.kv_pos = [dev(p, torch.int32) for p in pos_per_rank]
        if doc is not None:
            self.q_doc = [dev(doc[pos_per_rank[r]], torch.int32) for r in self.ranks]
            self.kv_doc = [dev(doc[p], torch.int32) for p in pos_per_rank]
        else:
            self.q_doc = self.kv_doc = None

    def alloc_fwd(self):
        B, hq, sq, d = self.q[0].shape
        self.o_acc = [torch.zeros(B, hq, sq, d, dtype=torch.float32, device="cuda") for _ in self.ranks]
        self.lse = [torch.zeros(B, hq, sq, dtype=torch.float32, device="cuda") for _ in self.ranks]
        self.out = [torch.empty_strided(q.shape, q.stride(), dtype=self.dt, device="cuda") for q in self.q]
        for o in self.out:
            o.fill_(float("nan"))

    def forward(self, flags=0, start_step=0, stop_step=0, copy_stream="side", alloc=True, workspace=None):
        if alloc:
            self.alloc_fwd()
        xs = torch.cuda.Stream() if copy_stream == "side" else None
        ra.ringattn_run(self.q, self.k, self.v, self.q_pos, self.kv_pos, o_acc=self.o_acc, lse=self.lse,
                        out=self.out, q_doc=self.q_doc, kv_doc=self.kv_doc, first_rank=self.ranks[0],
                        start_step=start_step, stop_step=stop_step, mask_mode=MASKS[self.mask],
                        pass_=ra.RA_PASS_FWD, flags=flags, copy_stream=xs, workspace=workspace)
        torch.cuda.synchronize()
        return self

    def backward(self, flags=0, copy_stream="side"):
        B, hq, sq, d = self.q[0].shape
        hkv, sk = self.k[0].shape[1], self.k[0].shape[2]
        self.delta = [torch.zeros(B, hq, sq, dtype=torch.float32, device="cuda") for _ in self.ranks]
        self.dq = [torch.zeros(B, hq, sq, d, dtype=torch.float32, device="cuda") for _ in self.ranks]
        self.dk = [torch.zeros(B, hkv, sk, d, dtype=torch.float32, device="cuda") for _ in range(self.n)]
        self.dv = [torch.zeros(B, hkv, sk, d, dtype=torch.float32, device="cuda") for _ in range(self.n)]
        xs = torch.cuda.Stream() if copy_stream == "side" else None
        ra.ringattn_run(self.q, self.k, self.v, self.q_pos, self.kv_pos, lse=self.lse, out=self.out,
                        q_doc=self.q_doc, kv_doc=self.kv_doc, d_o=self.do, delta=self.delta, dq=self.dq,
                        dk=self.dk, dv=self.dv, first_rank=self.ranks[0], mask_mode=MASKS[self.mask],
                        pass_=ra.RA_PASS_BWD, flags=flags, copy_stream=xs)
        torch.cuda.synchronize()
        return self

    def numpy(self, name):
        return [t.detach().float().cpu().numpy().astype(np.float64) for t in getattr(self, name)]


def oracle_rows(inp, rows, mask, doc=None, scale=None):
    """Oracle O, LSE of the queries at global indices `rows` against every key of the context.

    `inp["q"]` holds the query rows listed in `inp["q_rows"]` (global indices).
    """
    rows = np.asarray(rows)
    where = {int(g): i for i, g in enumerate(inp["q_rows"])}
    qsel = inp["q"][:, :, [where[int(g)] for g in rows]]
    s = inp["k"].shape[2]
    pos = np.arange(s)
    return oracle.attention_forward(qsel, inp["k"], inp["v"], rows, pos, mask,
                                    None if doc is None else doc[rows], doc, scale=scale,
                                    row_block=128, skip_masked_columns=mask != "none")


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def rel_l2(a, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(np.asarray(a, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300))
