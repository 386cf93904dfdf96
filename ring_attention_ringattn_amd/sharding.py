"""Sequence sharding of a ring: which global tokens each rank holds.

Host-side bookkeeping (no attention math).  A tensor sharded along the
sequence over N ranks is cut into N equal parts (Accelerate context-parallel
guide, technical details, definition of a shard): ``contiguous`` gives rank r
tokens [r S/N, (r+1) S/N).  ``zigzag`` cuts 2N chunks of c = S/2N tokens and
gives rank r chunk r followed by chunk 2N-1-r, which balances a causal mask:
every rank then has the same number of visible (query, key) pairs at every
step.  The positions returned are what the kernels mask with.
"""
from __future__ import annotations

import numpy as np


def shard_positions(seq: int, n: int, scheme: str) -> list:
    """int32 global positions of each rank's tokens, in the order the rank stores them."""
    if n < 1 or seq % n:
        raise ValueError(f"sequence of {seq} tokens does not split into {n} equal shards")
    if scheme == "contiguous":
        part = seq // n
        return [np.arange(r * part, (r + 1) * part, dtype=np.int32) for r in range(n)]
    if scheme == "zigzag":
        if seq % (2 * n):
            raise ValueError(f"zigzag needs {2 * n} equal chunks of {seq} tokens")
        c = seq // (2 * n)
        out = []
        for r in range(n):
            lo = np.arange(r * c, (r + 1) * c, dtype=np.int32)
            hi = np.arange((2 * n - 1 - r) * c, (2 * n - r) * c, dtype=np.int32)
            out.append(np.concatenate([lo, hi]))
        return out
    raise ValueError(f"unknown sharding scheme {scheme!r}")


def block_of(rank: int, step: int, n: int) -> int:
    """Block a rank attends to at a ring step: it received it after `step` hops from rank - step."""
    return (rank - step) % n


def causal_pairs_zigzag(n: int, c: int, rank: int, block: int) -> int:
    """Visible causal pairs of a zigzag rank's queries against one block (closed form)."""
    return 2 * c * c + (c if rank == block else 0)
