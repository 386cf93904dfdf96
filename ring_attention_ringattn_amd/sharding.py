"""Sequence sharding of a ring: which global tokens each rank holds.

Host-side bookkeeping (no attention math).  A tensor sharded along the
sequence over N ranks is cut into N equal parts (the Accelerate guide, "Context
Parallel no 🤗 accelerate", section "Detalhes técnicos", the definition of a
shard): ``contiguous`` gives rank r
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


# ---------------------------------------------------------------- model buffers
# Utilities for the tensors a training step feeds the attention: input ids,
# labels, masks.  They shard a buffer along its sequence dimension exactly as
# shard_positions shards the tokens, so a rank's buffer rows line up with the
# positions its kernels mask with.

def _index(x, dim, idx):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.index_select(dim, torch.as_tensor(idx, dtype=torch.long, device=x.device))
    except ImportError:      # pragma: no cover - torch is part of this package's environment
        pass
    return np.take(x, idx, axis=dim)


def shard_buffer(x, seq_dim: int, n: int, rank: int, scheme: str = "zigzag"):
    """Rank `rank`'s part of `x` along `seq_dim` (torch tensor or numpy array), in the
    order the rank stores its tokens (see shard_positions)."""
    return _index(x, seq_dim, shard_positions(x.shape[seq_dim], n, scheme)[rank])


def unshard_buffers(shards, seq_dim: int, scheme: str = "zigzag"):
    """Inverse of shard_buffer over all ranks: the buffer in global token order (what
    an all-gather along the sequence returns)."""
    n = len(shards)
    seq = sum(s.shape[seq_dim] for s in shards)
    order = np.concatenate(shard_positions(seq, n, scheme))
    inverse = np.empty_like(order)
    inverse[order] = np.arange(seq, dtype=order.dtype)
    try:
        import torch
        if isinstance(shards[0], torch.Tensor):
            return _index(torch.cat(list(shards), dim=seq_dim), seq_dim, inverse)
    except ImportError:      # pragma: no cover
        pass
    return _index(np.concatenate(shards, axis=seq_dim), seq_dim, inverse)


def shift_labels(labels, seq_dim: int = 1, ignore_index: int = -100):
    """Causal-LM targets: token t's label is token t+1, the last position gets
    `ignore_index`.  Shift BEFORE sharding (the Accelerate guide, section "Interface
    do Accelerate", on labels that are a copy of the input ids): a shard cannot see the first token of
    the next shard, so shifting after sharding misaligns every shard's last label."""
    try:
        import torch
        if isinstance(labels, torch.Tensor):
            out = torch.full_like(labels, ignore_index)
            n = labels.shape[seq_dim]
            out.narrow(seq_dim, 0, n - 1).copy_(labels.narrow(seq_dim, 1, n - 1))
            return out
    except ImportError:      # pragma: no cover
        pass
    out = np.full_like(labels, ignore_index)
    src = [slice(None)] * labels.ndim
    dst = [slice(None)] * labels.ndim
    src[seq_dim], dst[seq_dim] = slice(1, None), slice(0, -1)
    out[tuple(dst)] = labels[tuple(src)]
    return out


class maybe_context_parallel:
    """Context manager that shards torch buffers in place along their sequence
    dimension for the block (the Accelerate guide, sections "Como usar paralelismo de
    contexto?" and "Interface do Accelerate": the
    `maybe_context_parallel(buffers, buffer_seq_dims, no_restore_buffers)` pattern).

    It is a no-op when context parallelism is off (`n` is None or 1).  Otherwise,
    on entry every buffer's data is replaced by rank `rank`'s shard (the Python
    object stays the same, so references such as batch["input_ids"] see the
    shard); on exit every buffer not in `no_restore_buffers` gets its full data
    back (with one process per rank that is an all-gather; here the full tensor
    is kept).  Create a new one for every step: an instance can be entered once.
    """

    def __init__(self, buffers, buffer_seq_dims, no_restore_buffers=(), n=None, rank=0, scheme="zigzag"):
        if len(buffers) != len(buffer_seq_dims):
            raise ValueError("one sequence dimension per buffer")
        self.buffers, self.dims = list(buffers), list(buffer_seq_dims)
        self.no_restore = {id(b) for b in no_restore_buffers}
        self.n, self.rank, self.scheme = n, rank, scheme
        self._saved, self._used = None, False

    def __enter__(self):
        if self._used:
            raise RuntimeError("maybe_context_parallel instances are single-use: create one per step")
        self._used = True
        if self.n is None or self.n == 1:
            return self
        self._saved = [b.data for b in self.buffers]
        for b, d in zip(self.buffers, self.dims):
            b.data = shard_buffer(b.data, d, self.n, self.rank, self.scheme)
        return self

    def __exit__(self, *exc):
        if self._saved is not None:
            for b, full in zip(self.buffers, self._saved):
                if id(b) not in self.no_restore:
                    b.data = full
            self._saved = None
        return False
