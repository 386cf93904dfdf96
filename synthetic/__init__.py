"""Seeded synthetic inputs for ring attention.

This module is shared by the fp64 oracle's tests and by the GPU path's tests
and benchmark.  It only draws random numbers and describes workload shapes; it
holds none of the attention arithmetic (no scores, softmax, masks, sharding or
merging), so neither side can inherit a bug of the other from here.

Workloads (all in global token order, layout [B, H, S, D]):

* ``c1`` fp32, 2 heads (MHA), head_dim 64, S = 512, 4 contiguous shards,
  causal, N(0,1) values.
* ``c2`` bf16, 32 q heads / 8 kv heads, head_dim 128, S = 8192, 4 zigzag
  shards, causal, N(0,1)*0.5, forward only.
* ``c3`` bf16, one rank's share of a 131072-token context at 8 shards
  (16384 local queries, 8 key/value blocks of 16384), zigzag, causal.
* ``c4`` as c3 at 262144 tokens (32768 per shard), forward and backward,
  dO ~ N(0,1).
* ``c5`` bf16, 65536 packed tokens from lognormal document lengths
  (median 2048, sigma 1.2, clipped to [64, 32768]), document-causal mask,
  4 contiguous shards, forward and backward.

Value recipe.  Every tensor is made of blocks of ``ROW_BLOCK`` tokens of one
(batch, head); each block is drawn as float32 standard normals from its own
PCG64 stream seeded with ``SeedSequence([seed, tensor_tag, b, h, block])``,
multiplied by the workload's value scale and, for bf16 workloads, rounded to
the nearest bf16 value (ties to even).  Per-block streams let a test or the
benchmark materialise one shard's rows without drawing the rest of a
262144-token tensor.  Document lengths are drawn first, one standard normal at
a time, from ``default_rng(seed)``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

ROW_BLOCK = 128

TAG_Q, TAG_K, TAG_V, TAG_DO = 1, 2, 3, 4

# mask kinds, named by what they mean (each side maps these to its own codes)
MASK_NONE, MASK_CAUSAL, MASK_DOC_CAUSAL = "none", "causal", "doc_causal"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    batch: int
    hq: int
    hkv: int
    head_dim: int
    seq: int              # total tokens of the (packed) context
    n_shards: int         # ring size N
    sharding: str         # "contiguous" or "zigzag"
    mask: str             # MASK_*
    value_scale: float
    do_scale: float
    seed: int
    emulated_ranks: Optional[Sequence[int]]   # None = all N ranks
    backward: bool
    doc_lengths: bool = False                 # lognormal packed documents

    @property
    def shard_len(self) -> int:
        return self.seq // self.n_shards

    def ranks(self):
        return list(range(self.n_shards)) if self.emulated_ranks is None else list(self.emulated_ranks)


WORKLOADS = {
    "c1": Workload("c1", "f32", 1, 2, 2, 64, 512, 4, "contiguous", MASK_CAUSAL,
                   1.0, 1.0, 1, None, False),
    "c2": Workload("c2", "bf16", 1, 32, 8, 128, 8192, 4, "zigzag", MASK_CAUSAL,
                   0.5, 1.0, 2, None, False),
    "c3": Workload("c3", "bf16", 1, 32, 8, 128, 131072, 8, "zigzag", MASK_CAUSAL,
                   0.5, 1.0, 3, (0,), False),
    "c4": Workload("c4", "bf16", 1, 32, 8, 128, 262144, 8, "zigzag", MASK_CAUSAL,
                   0.5, 1.0, 4, (0,), True),
    "c5": Workload("c5", "bf16", 1, 32, 8, 128, 65536, 4, "contiguous", MASK_DOC_CAUSAL,
                   0.5, 1.0, 5, None, True, doc_lengths=True),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 value (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    Inputs here are finite normal draws, so NaN handling is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return rounded.view(np.float32)


def _block_stream(seed: int, tag: int, b: int, h: int, blk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, b, h, blk])))


def draw_rows(w: Workload, tag: int, heads: int, rows: np.ndarray, scale: float) -> np.ndarray:
    """Values of tensor ``tag`` at global token indices ``rows``: [B, heads, len(rows), D] float32."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((w.batch, heads, rows.size, w.head_dim), dtype=np.float32)
    if rows.size == 0:
        return out
    blk_of = rows // ROW_BLOCK
    order = np.argsort(blk_of, kind="stable")
    blocks, starts = np.unique(blk_of[order], return_index=True)
    ends = np.append(starts[1:], rows.size)
    for b in range(w.batch):
        for h in range(heads):
            for blk, s, e in zip(blocks, starts, ends):
                sel = order[s:e]
                vals = _block_stream(w.seed, tag, b, h, int(blk)).standard_normal(
                    (ROW_BLOCK, w.head_dim), dtype=np.float32)
                vals *= np.float32(scale)
                if w.dtype == "bf16":
                    vals = bf16_round(vals)
                out[b, h, sel] = vals[rows[sel] - blk * ROW_BLOCK]
    return out


def doc_lengths(seed: int, total: int, median: float = 2048.0, sigma: float = 1.2,
                lo: int = 64, hi: int = 32768) -> list:
    """Lognormal document lengths packed up to ``total`` tokens.

    Each length is round-half-even(exp(ln(median) + sigma*z)) clipped to
    [lo, hi], with z drawn one at a time from default_rng(seed); lengths are
    appended until they reach ``total`` and the last one is cut to fit.
    """
    rng = np.random.default_rng(seed)
    out, acc = [], 0
    while acc < total:
        z = rng.standard_normal()
        n = int(np.clip(np.round(np.exp(math.log(median) + sigma * z)), lo, hi))
        n = min(n, total - acc)
        out.append(n)
        acc += n
    return out


def cu_seqlens(w: Workload) -> Optional[np.ndarray]:
    """int32 [n_docs + 1] cumulative document offsets, or None without documents."""
    if not w.doc_lengths:
        return None
    lens = doc_lengths(w.seed, w.seq)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def make_inputs(w: Workload, q_rows: Optional[np.ndarray] = None, backward: Optional[bool] = None):
    """Global inputs of a workload.

    ``q_rows``: global token indices of the query rows to materialise (Q and
    dO); default all.  K and V always cover all ``w.seq`` tokens.
    Returns a dict with float32 arrays q, k, v (and do), plus cu_seqlens.
    """
    all_rows = np.arange(w.seq)
    q_rows = all_rows if q_rows is None else np.asarray(q_rows)
    back = w.backward if backward is None else backward
    d = {
        "q": draw_rows(w, TAG_Q, w.hq, q_rows, w.value_scale),
        "k": draw_rows(w, TAG_K, w.hkv, all_rows, w.value_scale),
        "v": draw_rows(w, TAG_V, w.hkv, all_rows, w.value_scale),
        "q_rows": q_rows,
        "cu_seqlens": cu_seqlens(w),
    }
    if back:
        d["do"] = draw_rows(w, TAG_DO, w.hq, q_rows, w.do_scale)
    return d


def small_workload(name: str, **over) -> Workload:
    """A reduced copy of a workload (for tests that must finish in seconds)."""
    return dataclasses.replace(WORKLOADS[name], **over)
