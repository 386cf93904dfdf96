"""Exhaustive Dynamic-CP planner: the optimum the product's heuristic solver is checked against.

TEST INFRASTRUCTURE (see the package header).  The problem is the one the
Dynamic-CP page ("Optimización del entrenamiento variable con Dynamic Context
Parallelism en Megatron Core", section "Modelado del programador de datos") gives
its solver: pack variable-length
sequences into micro-batches and choose a context-parallel size per
micro-batch so as to maximise efficiency without exceeding the GPU memory
limit.  Written out (the same readings the product documents):

* a micro-batch holding n tokens may use CP size c (a power of two up to the
  number of GPUs G) only if n <= c * tokens_per_gpu;
* it runs on an aligned group of c GPUs [k c, (k+1) c); its cost cost(docs, c)
  is charged to every GPU of the group;
* the iteration time is the largest per-GPU total; the planner minimises it.

Plain enumeration -- every set partition of the sequences, every feasible CP
size per part, every aligned group per part -- with one pruning rule (stop a
branch once it cannot beat the best plan found).  Only for a handful of
sequences.
"""
import math


def _partitions(items):
    """Every set partition of the list `items` (as lists of lists)."""
    if not items:
        yield []
        return
    first, rest = items[0], items[1:]
    for part in _partitions(rest):
        for k in range(len(part)):
            yield part[:k] + [[first] + part[k]] + part[k + 1:]
        yield [[first]] + part


def optimal_time(lengths, n_gpus, tokens_per_gpu, cost):
    """Smallest achievable iteration time, or inf if some sequence cannot fit."""
    sizes = []
    c = 1
    while c <= n_gpus:
        sizes.append(c)
        c *= 2
    best = math.inf
    for part in _partitions(list(range(len(lengths)))):
        blocks = []
        for p in part:
            tokens = sum(lengths[i] for i in p)
            opts = [(c, cost([lengths[i] for i in p], c)) for c in sizes if tokens <= c * tokens_per_gpu]
            if not opts:
                break
            blocks.append(opts)
        else:
            loads = [0.0] * n_gpus

            def place(b):
                nonlocal best
                if max(loads) >= best:
                    return
                if b == len(blocks):
                    best = max(loads)
                    return
                for c, t in blocks[b]:
                    for grp in range(n_gpus // c):
                        for g in range(grp * c, (grp + 1) * c):
                            loads[g] += t
                        place(b + 1)
                        for g in range(grp * c, (grp + 1) * c):
                            loads[g] -= t
            place(0)
    return best
