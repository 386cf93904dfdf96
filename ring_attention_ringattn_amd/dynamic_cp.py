"""Dynamic context parallelism: an attention cost model and a packing / CP-size solver.

Follows the Dynamic-CP page ("Optimización del entrenamiento variable con Dynamic
Context Parallelism en Megatron Core"), sections "Modelado del programador de
datos" and "Colaboración del modelo de costos, solucionador y simulador": a cost
model estimates each sample's run time from its sequence
length (attention work grows with the square of the length), and a solver
uses it to pack variable-length sequences into micro-batches and to choose a
context-parallel size per micro-batch, maximising efficiency without
exceeding the GPU memory limit.  The page's third component, a pipeline
simulator, belongs to pipeline parallelism and is not built here.

The page gives no formulas; the readings taken here:

* Cost of one micro-batch (documents d_1..d_k packed in THD form in that order,
  document-causal attention, split contiguously over a ring of c ranks):
      T = alpha * P_crit + beta * sum d_i / c + eps * sum d_i + gamma * c + delta
  P_crit is the attention work on the ring's critical path: every ring step
  ends when its slowest rank does, so P_crit = sum over steps t of the largest,
  over ranks r, count of visible (query, key) pairs between rank r's queries and
  the block it holds at step t (`step_pairs`, exact, from the document
  boundaries).  For balanced work it is the quadratic sum d_i^2 / (2c) the page
  speaks of; for one long document split contiguously the last rank does
  (2c - 1) / c times the mean, and P_crit charges that.  beta: linear work split
  over c; eps: the work every ring step repeats on the rank's running output
  (c steps over n/c rows: n rows whatever c is); gamma per ring step (c steps)
  and a fixed delta.  The coefficients are fitted by least squares to timings
  of this library's own kernels (`measure`), each micro-batch timed the same
  way: the sum over steps of its slowest rank's step time.
* Memory limit: at most `tokens_per_gpu` tokens of a micro-batch per GPU, so a
  micro-batch of n tokens needs c >= n / tokens_per_gpu; c is a power of two
  up to the number of GPUs (the page builds CP groups of power-of-two sizes).
* Iteration time of a plan: every micro-batch runs on an aligned group of c
  GPUs; a GPU's load is the sum of the costs of the micro-batches it takes
  part in; the iteration takes as long as the most loaded GPU (data-parallel
  ranks wait for each other at the gradient synchronisation, the imbalance
  the page describes).
* Baseline ("packing only", the reference of the page's Table 1, section
  "Resultados de benchmarks"): one static CP size,
  set by the longest sequence, for every micro-batch; sequences packed to the
  same token budget.

Host code; `measure` alone uses the GPU (through the library's ring driver).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Sequence, Tuple

import numpy as np


TILE = 64   # a ring rank holds whole 64-token tiles; a micro-batch is padded to that


def ring_docs(docs: Sequence[int], cp: int) -> List[int]:
    """The documents of a micro-batch as its ring runs them: one extra padding document
    makes the packed stream a whole number of 64-token tiles per rank."""
    pad = (-int(sum(docs))) % (TILE * cp)
    return [int(x) for x in docs] + ([pad] if pad else [])


def step_pairs(docs: Sequence[int], cp: int) -> np.ndarray:
    """[cp, cp] int64: visible (query, key) pairs of rank r's queries against the block it
    holds at ring step t, block (r - t) mod cp (document-causal; the padded stream split
    contiguously).  For queries i in [qa, qb) and keys [ka, ka + L) of one document, the
    count is sum_i clamp(i - ka + 1, 0, L), a difference of two closed-form prefix sums."""
    d = np.asarray(ring_docs(docs, cp), dtype=np.int64)
    ends = np.cumsum(d)
    starts = ends - d
    s = int(ends[-1]) // cp
    r = np.arange(cp)[:, None, None]
    t = np.arange(cp)[None, :, None]
    j = (r - t) % cp
    qa, qb = np.maximum(starts, r * s), np.minimum(ends, (r + 1) * s)
    ka, kb = np.maximum(starts, j * s), np.minimum(ends, (j + 1) * s)
    L = np.maximum(kb - ka, 0)

    def prefix(x):   # sum over queries i < x of the keys of [ka, ka + L) at or before i
        m = np.maximum(x - ka, 0)
        inside = np.minimum(m, L)
        return inside * (inside + 1) // 2 + np.maximum(m - L, 0) * L
    pairs = np.where(qb > qa, prefix(qb) - prefix(qa), 0)
    return pairs.sum(axis=2)


def critical_pairs(docs: Sequence[int], cp: int) -> int:
    """Attention pairs on the ring's critical path: each step waits for its slowest rank."""
    return int(step_pairs(docs, cp).max(axis=0).sum())


@dataclasses.dataclass(frozen=True)
class CostModel:
    alpha: float    # ms per visible (query, key) pair on the critical path (all heads)
    beta: float     # ms per token, split over c
    eps: float      # ms per token of the micro-batch, not split (per-step running output)
    gamma: float    # ms per ring step
    delta: float    # ms fixed

    def predict(self, docs: Sequence[int], cp: int) -> float:
        n = float(sum(docs))
        return float(self.alpha * critical_pairs(docs, cp) + self.beta * n / cp + self.eps * n + self.gamma * cp
                     + self.delta)


def fit_cost_model(samples: Sequence[Tuple[Sequence[int], int, float]]) -> Tuple[CostModel, float]:
    """Non-negative least-squares fit of (alpha, beta, eps, gamma, delta) to (docs, cp, measured ms)
    samples, weighted by 1/ms so that every sample counts by its relative error; every term is a
    cost, so none may come out negative.  Returns the model and the largest relative error over
    the samples."""
    from scipy.optimize import nnls
    rows, y = [], []
    for docs, cp, ms in samples:
        n = float(sum(docs))
        rows.append([critical_pairs(docs, cp), n / cp, n, cp, 1.0])
        y.append(ms)
    a, y = np.asarray(rows), np.asarray(y)
    w = 1.0 / y
    # columns scaled to unit norm for the solver's conditioning (pairs ~1e9, tokens ~1e4, cp ~1)
    aw = a * w[:, None]
    norm = np.linalg.norm(aw, axis=0)
    norm[norm == 0] = 1.0
    coef, _ = nnls(aw / norm, y * w)
    model = CostModel(*[float(x) for x in coef / norm])
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

@dataclasses.dataclass
class RingTiming:
    ms: float                 # forward + backward of the ring: per step, its slowest rank
    per_rank_ms: List[float]  # each rank's own forward + backward ring


def time_micro_batch(docs: Sequence[int], cp: int, hq: int = 32, hkv: int = 8, d: int = 128, reps: int = 5,
                     seed: int = 0) -> RingTiming:
    """Forward + backward attention of one packed micro-batch (documents `docs`, document-
    causal, contiguous shards) on a ring of `cp` ranks, as a real ring would take it.

    Every rank runs alone on this GPU through the library's ring driver (one emulated rank
    per call), with events around each of its ring steps and around the whole call.  A ring
    step ends when its slowest rank does, so the ring's time is the sum over steps of the
    largest step time over ranks, plus the largest per-rank time outside the steps (tile
    tables, backward preprocess, launch gaps); forward and backward each.  Each (rank,
    step) time is the median over `reps` runs."""
    import torch
    import ring_attention_ringattn_amd as ra
    from . import sharding

    docs = ring_docs(docs, cp)
    total = int(sum(docs))
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
    ws = torch.empty(max(ra.ringattn_run_workspace_size(q[0], k[0], cp, 1, pass_=p_, mask_mode=ra.RA_MASK_DOC_CAUSAL)
                         for p_ in (ra.RA_PASS_FWD, ra.RA_PASS_BWD)), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()

    def events(n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in ev:
            e.record()   # creates the underlying event
        return ev

    def run_rank(r, ev_f, ev_b, call):
        one = dict(q_doc=[doc[r]], kv_doc=doc, first_rank=r, mask_mode=ra.RA_MASK_DOC_CAUSAL, workspace=ws,
                   copy_stream=side)
        call[0].record()
        ra.ringattn_run([q[r]], k, v, [qp[r]], qp, o_acc=[o_acc[r]], lse=[lse[r]], out=[out[r]],
                        step_events=[e.cuda_event for e in ev_f], **one)
        call[1].record()
        ra.ringattn_run([q[r]], k, v, [qp[r]], qp, lse=[lse[r]], out=[out[r]], d_o=[do[r]], delta=[delta[r]],
                        dq=[dq[r]], dk=dk, dv=dv, pass_=ra.RA_PASS_BWD, step_events=[e.cuda_event for e in ev_b],
                        **one)
        call[2].record()

    sets = [[(events(2 * cp), events(2 * cp), events(3)) for _ in range(cp)] for _ in range(reps + 1)]
    for rep in range(reps + 1):   # the first round is a warm-up
        for r in range(cp):
            run_rank(r, *sets[rep][r])
    torch.cuda.synchronize()
    # [reps, cp ranks, cp steps] step times and [reps, cp] time outside the steps, per pass
    step = np.zeros((2, reps, cp, cp))
    rest = np.zeros((2, reps, cp))
    for rep in range(reps):
        for r in range(cp):
            ev_f, ev_b, call = sets[rep + 1][r]
            for pss, ev in ((0, ev_f), (1, ev_b)):
                step[pss, rep, r] = [ev[2 * t].elapsed_time(ev[2 * t + 1]) for t in range(cp)]
                rest[pss, rep, r] = call[pss].elapsed_time(call[pss + 1]) - step[pss, rep, r].sum()
    med_step, med_rest = np.median(step, axis=1), np.median(rest, axis=1)   # [2, cp, cp], [2, cp]
    ring = float(sum(med_step[p_].max(axis=0).sum() + med_rest[p_].max() for p_ in range(2)))
    per_rank = [float(med_step[:, r].sum() + med_rest[:, r].sum()) for r in range(cp)]
    return RingTiming(ring, per_rank)


def measure(grid_tokens=(8192, 16384, 32768), doc_lengths=(512, 2048, 8192, 32768), cps=(1, 2, 4, 8), **timing):
    """Timings for the cost-model fit: micro-batches of equal documents, every CP size
    (`timing`: head counts, head_dim, reps of `time_micro_batch`)."""
    samples = []
    for tot in grid_tokens:
        for dl in doc_lengths:
            if dl > tot:
                continue
            docs = [dl] * (tot // dl)
            for c in cps:
                if tot // c < TILE:
                    continue
                samples.append((docs, c, time_micro_batch(docs, c, **timing).ms))
    return samples


def execute(plan: Plan, lengths: Sequence[int], n_gpus: int, **timing) -> float:
    """Measured iteration time of a plan: every micro-batch is timed on this GPU at its CP
    size (`time_micro_batch`: the ring's slowest-rank critical path) and charged to the
    GPUs of its group."""
    loads = [0.0] * n_gpus
    for mb in plan.micro_batches:
        t = time_micro_batch([lengths[i] for i in mb.seqs], mb.cp, **timing).ms
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
    mean_err = float(np.mean([abs(model.predict(d, c) - ms) / ms for d, c, ms in samples]))
    lengths = lognormal_lengths(args.seed, args.sequences)
    dyn = solve_dynamic(lengths, args.gpus, args.tokens_per_gpu, model)
    sta = solve_static(lengths, args.gpus, args.tokens_per_gpu, model)
    for p in (dyn, sta):
        check_plan(p, lengths, args.gpus, args.tokens_per_gpu)
    t_dyn, t_sta = execute(dyn, lengths, args.gpus), execute(sta, lengths, args.gpus)
    print(json.dumps({
        "timing": "per micro-batch: sum over ring steps of the slowest rank's step time, forward + backward",
        "cost_model": dataclasses.asdict(model), "fit_samples": len(samples), "fit_max_rel_err": round(err, 4),
        "fit_mean_rel_err": round(mean_err, 4),
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
