"""Ring attention emulated in fp64: shard, attend block by block, merge.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

This is the method written in the pages' order, used only to check the
method itself against the plain definition in ``attention.py``:

* Sequence sharding: a tensor sharded along a dimension over N ranks is cut
  into N equal parts (the Accelerate guide, "Context Parallel no 🤗 accelerate",
  section "Detalhes técnicos", the definition of a shard).  The zigzag variant
  cuts 2N equal chunks and gives
  rank r chunks r and 2N-1-r; it is not on the pages and is the usual
  load-balanced reading for causal masks.
* Each rank keeps its Q shard, attends first to its own K/V block, then to
  every other rank's block once, each block arriving from the previous rank
  of the ring (same guide, section "Então, como funciona?" and its
  ring-rotation paragraph; the NVSHMEM page, "Optimización en el entrenamiento
  de modelos de lenguaje de largo contexto con NVSHMEM en JAX y XLA", section
  "Paralelismo de contexto y atención en anillo": send KV to the next device,
  compute incrementally while blocks circulate).  At step t rank r
  holds block (r - t) mod N.
* The per-block partial results are combined; the pages leave ``combine``
  undefined.  The reading taken: the exact log-sum-exp merge of normalised
  partials (O_a, LSE_a) (+) (O_b, LSE_b), with LSE = logaddexp(LSE_a, LSE_b)
  and O = exp(LSE_a - LSE) O_a + exp(LSE_b - LSE) O_b.  An empty partial
  (O = 0, LSE = -inf) is its identity.  It is the only combine that keeps
  the result equal to standard attention (NVSHMEM/XLA page, ring attention
  section).
"""
from __future__ import annotations

import numpy as np

from .attention import attention_forward


def shard_rows(seq, n, scheme):
    """Global token indices of each rank's shard, in the order the rank stores them."""
    if seq % n:
        raise ValueError("sequence length must divide evenly over the ranks")
    if scheme == "contiguous":
        part = seq // n
        return [np.arange(r * part, (r + 1) * part) for r in range(n)]
    if scheme == "zigzag":
        if seq % (2 * n):
            raise ValueError("zigzag needs 2N equal chunks")
        c = seq // (2 * n)
        return [np.concatenate([np.arange(r * c, (r + 1) * c),
                                np.arange((2 * n - 1 - r) * c, (2 * n - r) * c)]) for r in range(n)]
    raise ValueError(f"unknown sharding {scheme!r}")


def merge(o_a, lse_a, o_b, lse_b):
    """(O_a, LSE_a) (+) (O_b, LSE_b), exact; -inf LSE is the identity."""
    lse = np.logaddexp(lse_a, lse_b)
    fin = np.isfinite(lse)
    safe = np.where(fin, lse, 0.0)
    w_a = np.where(np.isfinite(lse_a) & fin, np.exp(np.where(np.isfinite(lse_a), lse_a, 0.0) - safe), 0.0)
    w_b = np.where(np.isfinite(lse_b) & fin, np.exp(np.where(np.isfinite(lse_b), lse_b, 0.0) - safe), 0.0)
    o = w_a[..., None] * o_a + w_b[..., None] * o_b
    return o, lse


def ring_forward(q, k, v, pos, mode, n, scheme, doc=None, scale=None, step_order=None):
    """Attention of every rank's Q shard over the N circulating K/V blocks.

    Inputs are global tensors [B,H,S,D]; ``pos``/``doc`` give each token's
    global position and document.  Returns O, LSE in global order, so that
    the result can be compared with ``attention_forward`` on whole tensors.
    ``step_order(r, n)`` may return another visiting order of the blocks.
    """
    q = np.asarray(q, dtype=np.float64)
    B, hq, s, d = q.shape
    shards = shard_rows(s, n, scheme)
    o_all = np.zeros((B, hq, s, d))
    lse_all = np.full((B, hq, s), -np.inf)
    pos = np.asarray(pos)
    for r in range(n):
        qi = shards[r]
        o_acc = np.zeros((B, hq, qi.size, d))
        lse_acc = np.full((B, hq, qi.size), -np.inf)
        order = [(r - t) % n for t in range(n)] if step_order is None else step_order(r, n)
        for j in order:
            kj = shards[j]
            o_t, lse_t = attention_forward(
                q[:, :, qi], np.asarray(k)[:, :, kj], np.asarray(v)[:, :, kj], pos[qi], pos[kj], mode,
                None if doc is None else np.asarray(doc)[qi], None if doc is None else np.asarray(doc)[kj],
                scale=scale)
            o_acc, lse_acc = merge(o_acc, lse_acc, o_t, lse_t)
        o_all[:, :, qi] = o_acc
        lse_all[:, :, qi] = lse_acc
    return o_all, lse_all
