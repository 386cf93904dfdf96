"""Dynamic context parallelism: an attention cost model and a packing / CP-size solver.

Follows the Dynamic-CP page (Megatron Core), section on modelling the data
scheduler: a cost model estimates each sample's run time from its sequence
length (attention work grows with the square of the length), and a solver
uses it to pack variable-length sequences into micro-batches and to choose a
context-parallel size per micro-batch, maximising efficiency without
exceeding the GPU memory limit.  The page's third component, a pipeline
simulator, belongs to pipeline parallelism and is not built here.

The page gives no formulas; the readings taken here:

* Cost of one micro-batch (documents d_1..d_k packed in THD form, document-
  causal attention, context-parallel size c, per rank):
      T = (alpha * sum d_i^2 + beta * sum d_i) / c + eps * sum d_i + gamma * c + delta
  the quadratic and linear attention terms split over c ranks; eps for the work
  every ring step repeats on the rank's running output (c steps over n/c rows:
  n rows whatever c is); gamma per ring step (c steps) and a fixed delta.  The
  coefficients are fitted by least squares to timings of this library's own
  kernels (`measure`).
* Memory limit: at most `tokens_per_gpu` tokens of a micro-batch per GPU, so a
  micro-batch of n tokens needs c >= n / tokens_per_gpu; c is a power of two
  up to the number of GPUs (the page builds CP groups of power-of-two sizes).
* Iteration time of a plan: every micro-batch runs on an aligned group of c
  GPUs; a GPU's load is the sum of the costs of the micro-batches it takes
  part in; the iteration takes as long as the most loaded GPU (data-parallel
  ranks wait for each other at the gradient synchronisation, the imbalance
  the page describes).
* Baseline ("packing only", the page's Table 1 reference): one static CP size,
  set by the longest sequence, for every micro-batch; sequences packed to the
  same token budget.

Host code; `measure` alone uses the GPU (through the library's ring driver).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Sequence, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class CostModel:
    alpha: float    # ms per (token^2) of attention work, per rank before the split over c
    beta: float     # ms per token, split over c
    eps: float      # ms per token of the micro-batch, not split (per-step running output)
    gamma: float    # ms per ring step
    delta: float    # ms fixed

    def predict(self, docs: Sequence[int], cp: int) -> float:
        d = np.asarray(docs, dtype=np.float64)
        return float((self.alpha * np.sum(d * d) + self.beta * np.sum(d)) / cp + self.eps * np.sum(d)
                     + self.gamma * cp + self.delta)


def fit_cost_model(samples: Sequence[Tuple[Sequence[int], int, float]]) -> Tuple[CostModel, float]:
    """Least-squares fit of (alpha, beta, eps, gamma, delta) to (docs, cp, measured ms) samples,
    weighted by 1/ms so that every sample counts by its relative error.  Returns the model
    and the largest relative error over the samples."""
    rows, y = [], []
    for docs, cp, ms in samples:
        d = np.asarray(docs, dtype=np.float64)
        rows.append([np.sum(d * d) / cp, np.sum(d) / cp, np.sum(d), cp, 1.0])
        y.append(ms)
    a, y = np.asarray(rows), np.asarray(y)
    w = 1.0 / y
    coef, *_ = np.linalg.lstsq(a * w[:, None], y * w, rcond=None)
    model = CostModel(*[float(x) for x in coef])
    err = max(abs(model.predict(docs, cp) - ms) / ms for docs, cp, ms in samples)
    return model, err


@dataclasses.dataclass
class MicroBatch:
    seqs: List[int]     # indices into the length list
    cp: int
    group: int = -1     # aligned GPU group: GPUs [group * cp, (group + 1) * cp)


@dataclasses.dataclass
class Plan:
    micro_batches: List[MicroBatch]
    loads: List[float]  # per-GPU predicted load, ms

    @property
    def time(self) -> float:
        return max(self.loads)


def cp_needed(tokens: int, tokens_per_gpu: int, n_gpus: int) -> int:
    """Smallest power-of-two CP size that holds `tokens` under the memory limit."""
    c = 1
    while c * tokens_per_gpu < tokens:
        c *= 2
    if c > n_gpus:
        raise ValueError(f"{tokens} tokens do not fit on {n_gpus} GPUs of {tokens_per_gpu} tokens")
    return c


def _pack_ffd(order: Sequence[int], lengths: Sequence[int], capacity: int) -> List[List[int]]:
    """First-fit decreasing: sequences (already in decreasing order) into bins of `capacity` tokens."""
    bins: List[List[int]] = []
    used: List[int] = []
    for i in order:
        for b, u in enumerate(used):
            if u + lengths[i] <= capacity:
                bins[b].append(i)
                used[b] += lengths[i]
                break
        else:
            bins.append([i])
            used.append(lengths[i])
    return bins


def schedule(mbs: List[MicroBatch], lengths: Sequence[int], n_gpus: int, model: CostModel) -> Plan:
    """Longest-processing-time-first onto aligned GPU groups: each micro-batch, in
    decreasing predicted cost, goes to the group of its CP size whose busiest GPU is least
    loaded.  Sets every micro-batch's group; returns the plan with per-GPU loads."""
    loads = [0.0] * n_gpus
    cost = [model.predict([lengths[i] for i in mb.seqs], mb.cp) for mb in mbs]
    for k in sorted(range(len(mbs)), key=lambda k: -cost[k]):
        mb = mbs[k]
        best, best_load = 0, math.inf
        for grp in range(n_gpus // mb.cp):
            m = max(loads[grp * mb.cp:(grp + 1) * mb.cp])
            if m < best_load:
                best, best_load = grp, m
        mb.group = best
        for gpu in range(best * mb.cp, (best + 1) * mb.cp):
            loads[gpu] += cost[k]
    return Plan(mbs, loads)


def solve_dynamic(lengths: Sequence[int], n_gpus: int, tokens_per_gpu: int, model: CostModel) -> Plan:
    """Dynamic-CP plan, greedy: sequences in decreasing cost; each one either joins an
    existing micro-batch (at its CP size if the tokens fit, else at the smallest larger
    CP size, moving it to a group of that size), or opens a new micro-batch at the
    smallest CP size that holds it, placed on the aligned GPU
    group whose busiest GPU is least loaded -- whichever choice leaves the most loaded GPU
    least loaded (ties: the least total GPU time).  A short sequence thus runs on a small
    CP group unless joining a larger one balances the GPUs better.  The micro-batches are
    then re-placed longest-first (`schedule`) and the better placement is kept."""
    order = sorted(range(len(lengths)), key=lambda i: -model.predict([lengths[i]], 1))
    mbs: List[MicroBatch] = []
    cost: List[float] = []
    tokens: List[int] = []
    loads = [0.0] * n_gpus
    for i in order:
        n = lengths[i]
        c0 = cp_needed(n, tokens_per_gpu, n_gpus)
        # option A: a new micro-batch on the best group of CP size c0
        t_new = model.predict([n], c0)
        best_grp, best_grp_max = 0, math.inf
        for grp in range(n_gpus // c0):
            m = max(loads[grp * c0:(grp + 1) * c0])
            if m < best_grp_max:
                best_grp, best_grp_max = grp, m
        best = (max(max(loads), best_grp_max + t_new), t_new * c0, -1, best_grp)
        # option B: join micro-batch k, at its CP size if the tokens fit, else at the
        # smallest larger one (the micro-batch then moves to a group of that size)
        for k, mb in enumerate(mbs):
            merged = [lengths[j] for j in mb.seqs] + [n]
            c1 = cp_needed(tokens[k] + n, tokens_per_gpu, n_gpus) if tokens[k] + n <= n_gpus * tokens_per_gpu else 0
            if c1 == 0:
                continue
            c1 = max(c1, mb.cp)
            t = model.predict(merged, c1)
            lo, hi = mb.group * mb.cp, (mb.group + 1) * mb.cp
            if c1 == mb.cp:
                d = t - cost[k]
                ms = max(max(loads[:lo], default=0.0), max(loads[hi:], default=0.0), max(loads[lo:hi]) + d)
                cand = (ms, d * mb.cp, k, mb.group)
            else:
                tent = loads[:lo] + [x - cost[k] for x in loads[lo:hi]] + loads[hi:]
                g1, g1_max = 0, math.inf
                for grp in range(n_gpus // c1):
                    m = max(tent[grp * c1:(grp + 1) * c1])
                    if m < g1_max:
                        g1, g1_max = grp, m
                ms = max(max(tent), g1_max + t)
                cand = (ms, t * c1 - cost[k] * mb.cp, k, g1)
            if cand[:2] < best[:2]:
                best = cand[:3] + (cand[3],)
        k = best[2]
        if k < 0:
            mbs.append(MicroBatch([i], c0, best_grp))
            cost.append(t_new)
            tokens.append(n)
            for g in range(best_grp * c0, (best_grp + 1) * c0):
                loads[g] += t_new
        else:
            mb = mbs[k]
            for g in range(mb.group * mb.cp, (mb.group + 1) * mb.cp):
                loads[g] -= cost[k]
            mb.seqs.append(i)
            tokens[k] += n
            mb.cp = max(mb.cp, cp_needed(tokens[k], tokens_per_gpu, n_gpus))
            mb.group = best[3]
            cost[k] = model.predict([lengths[j] for j in mb.seqs], mb.cp)
            for g in range(mb.group * mb.cp, (mb.group + 1) * mb.cp):
                loads[g] += cost[k]
    greedy = Plan(mbs, loads)
    replaced = schedule([MicroBatch(list(mb.seqs), mb.cp) for mb in mbs], lengths, n_gpus, model)
    return replaced if replaced.time < greedy.time else greedy


def solve_static(lengths: Sequence[int], n_gpus: int, tokens_per_gpu: int, model: CostModel) -> Plan:
    """Packing only: one CP size for every micro-batch, set by the longest sequence, and
    sequences packed first-fit decreasing up to that CP group's token budget."""
    c = max(cp_needed(n, tokens_per_gpu, n_gpus) for n in lengths)
    order = sorted(range(len(lengths)), key=lambda i: -lengths[i])
    mbs = [MicroBatch(b, c) for b in _pack_ffd(order, lengths, c * tokens_per_gpu)]
    return schedule(mbs, lengths, n_gpus, model)


def check_plan(plan: Plan, lengths: Sequence[int], n_gpus: int, tokens_per_gpu: int) -> None:
    """Raise if a plan breaks a constraint: every sequence exactly once, memory limit,
    power-of-two CP size, aligned group inside the machine."""
    seen = sorted(i for mb in plan.micro_batches for i in mb.seqs)
    if seen != list(range(len(lengths))):
        raise AssertionError("every sequence must be in exactly one micro-batch")
    for mb in plan.micro_batches:
        if mb.cp < 1 or mb.cp & (mb.cp - 1) or mb.cp > n_gpus:
            raise AssertionError(f"bad CP size {mb.cp}")
        if sum(lengths[i] for i in mb.seqs) > mb.cp * tokens_per_gpu:
            raise AssertionError("memory limit exceeded")
        if not 0 <= mb.group < n_gpus // mb.cp:
            raise AssertionError("group outside the machine")


def lognormal_lengths(seed: int, n: int, median: float = 2048.0, sigma: float = 1.2, lo: int = 64,
                      hi: int = 32768) -> List[int]:
    """A synthetic variable-length batch: lognormal lengths clipped to [lo, hi] (the shape
    of the length distributions the page describes; its datasets are not used)."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in np.clip(np.round(np.exp(np.log(median) + sigma * rng.standard_normal(n))), lo, hi)]


# ------------------------------------------------------------------ measurement (GPU)

def time_micro_batch(docs: Sequence[int], cp: int, hq: int = 32, hkv: int = 8, d: int = 128, reps: int = 5,
                     seed: int = 0) -> float:
    """Per-rank milliseconds of forward + backward attention of one packed micro-batch
    (documents `docs`, document-causal) over a ring of `cp` ranks: all `cp` ranks are run
    on this GPU by the library's ring driver, and the time (median over `reps` runs) is
    divided by `cp`."""
    import torch
    import ring_attention_ringattn_amd as ra
    from . import sharding

    total = int(sum(docs))
    pad = (-total) % (64 * cp)             # whole 64-token tiles per rank; padding is its own document
    docs = list(docs) + ([pad] if pad else [])
    total += pad
    cu = torch.tensor(np.concatenate([[0], np.cumsum(docs)]).astype(np.int32), device="cuda")
    pos = sharding.shard_positions(total, cp, "contiguous")
    g = torch.Generator(device="cuda").manual_seed(seed)
    mk = lambda h: (torch.randn(1, h, total // cp, d, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    q = [mk(hq) for _ in range(cp)]
    k = [mk(hkv) for _ in range(cp)]
    v = [mk(hkv) for _ in range(cp)]
    do = [mk(hq) for _ in range(cp)]
    qp = [torch.from_numpy(p).cuda() for p in pos]
    doc = [ra.ringattn_docs_from_cu_seqlens(cu, int(p[0]), p.size) for p in pos]
    o_acc = [torch.empty(x.shape, device="cuda") for x in q]
    lse = [torch.empty(x.shape[:3], device="cuda") for x in q]
    out = [torch.empty_like(x) for x in q]
    delta = [torch.empty(x.shape[:3], device="cuda") for x in q]
    dq = [torch.zeros(x.shape, device="cuda") for x in q]
    dk = [torch.zeros(x.shape, device="cuda") for x in k]
    dv = [torch.zeros(x.shape, device="cuda") for x in k]
    ws = torch.empty(ra.ringattn_run_workspace_size(q[0], k[0], cp, cp, pass_=ra.RA_PASS_BWD,
                                                    mask_mode=ra.RA_MASK_DOC_CAUSAL), dtype=torch.uint8,
                     device="cuda")
    side = torch.cuda.Stream()

    def step():
        ra.ringattn_run(q, k, v, qp, qp, o_acc=o_acc, lse=lse, out=out, q_doc=doc, kv_doc=doc,
                        mask_mode=ra.RA_MASK_DOC_CAUSAL, workspace=ws, copy_stream=side)
        ra.ringattn_run(q, k, v, qp, qp, lse=lse, out=out, d_o=do, q_doc=doc, kv_doc=doc, delta=delta, dq=dq,
                        dk=dk, dv=dv, mask_mode=ra.RA_MASK_DOC_CAUSAL, pass_=ra.RA_PASS_BWD, workspace=ws,
                        copy_stream=side)
    step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for r in range(reps):
        step()
        ev[r + 1].record()
    torch.cuda.synchronize()
    return float(np.median([ev[r].elapsed_time(ev[r + 1]) for r in range(reps)])) / cp


def measure(grid_tokens=(8192, 16384, 32768), doc_lengths=(512, 2048, 8192, 32768), cps=(1, 2, 4, 8)):
    """Timings for the cost-model fit: micro-batches of equal documents, every CP size."""
    samples = []
    for tot in grid_tokens:
        for dl in doc_lengths:
            if dl > tot:
                continue
            docs = [dl] * (tot // dl)
            for c in cps:
                if tot // c < 64:
                    continue
                samples.append((docs, c, time_micro_batch(docs, c)))
    return samples


def execute(plan: Plan, lengths: Sequence[int], n_gpus: int) -> float:
    """Measured iteration time of a plan: every micro-batch is timed on this GPU at its CP
    size (`time_micro_batch`) and charged to the GPUs of its group."""
    loads = [0.0] * n_gpus
    for mb in plan.micro_batches:
        t = time_micro_batch([lengths[i] for i in mb.seqs], mb.cp)
        for g in range(mb.group * mb.cp, (mb.group + 1) * mb.cp):
            loads[g] += t
    return max(loads)


def main(argv=None):
    import argparse
    import json
    ap = argparse.ArgumentParser(description="Fit the attention cost model on this GPU and compare the "
                                             "Dynamic-CP plan with static packing, predicted and measured.")
    ap.add_argument("--gpus", type=int, default=8, help="GPUs the plan is made for (the ring is emulated)")
    ap.add_argument("--tokens-per-gpu", type=int, default=16384)
    ap.add_argument("--sequences", type=int, default=64)
    ap.add_argument("--seed", type=int, default=5)
    args = ap.parse_args(argv)
    samples = measure()
    model, err = fit_cost_model(samples)
    lengths = lognormal_lengths(args.seed, args.sequences)
    dyn = solve_dynamic(lengths, args.gpus, args.tokens_per_gpu, model)
    sta = solve_static(lengths, args.gpus, args.tokens_per_gpu, model)
    for p in (dyn, sta):
        check_plan(p, lengths, args.gpus, args.tokens_per_gpu)
    t_dyn, t_sta = execute(dyn, lengths, args.gpus), execute(sta, lengths, args.gpus)
    print(json.dumps({
        "cost_model": dataclasses.asdict(model), "fit_samples": len(samples), "fit_max_rel_err": round(err, 4),
        "worst_fit": sorted(([len(d), d[0], c, round(ms, 3), round(model.predict(d, c), 3)] for d, c, ms in samples),
                            key=lambda r: -abs(r[4] - r[3]) / r[3])[:6],
        "batch": {"sequences": len(lengths), "tokens": int(sum(lengths)), "longest": max(lengths),
                  "median_target": 2048, "seed": args.seed},
        "gpus": args.gpus, "tokens_per_gpu": args.tokens_per_gpu,
        "dynamic": {"micro_batches": len(dyn.micro_batches),
                    "cp_sizes": sorted({mb.cp for mb in dyn.micro_batches}),
                    "predicted_ms": round(dyn.time, 3), "measured_ms": round(t_dyn, 3)},
        "static": {"micro_batches": len(sta.micro_batches), "cp": sta.micro_batches[0].cp,
                   "predicted_ms": round(sta.time, 3), "measured_ms": round(t_sta, 3)},
        "speedup_predicted": round(sta.time / dyn.time, 3), "speedup_measured": round(t_sta / t_dyn, 3)}),
        flush=True)


if __name__ == "__main__":
    main()
