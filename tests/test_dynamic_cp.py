"""Dynamic-CP cost model and solver (host): fit, plan constraints, and the heuristic against
the exhaustive optimum of oracle/dynamic_cp.py on small instances."""
from functools import lru_cache

import numpy as np
import pytest

from oracle.dynamic_cp import optimal_time
from ring_attention_ringattn_amd import dynamic_cp as dcp

MODEL = dcp.CostModel(alpha=4e-8, beta=1e-4, eps=2e-6, gamma=0.05, delta=0.1)


@lru_cache(maxsize=None)
def _critical(docs, c):
    """Pairs on the ring's critical path, counted query token by query token: the packed
    stream padded to whole 64-token tiles per rank (the padding its own document), split
    contiguously; at step t rank r holds block (r - t) mod c; a query sees the keys of its
    own document at or before it; each step counts its busiest rank."""
    pad = (-sum(docs)) % (64 * c)
    lens = list(docs) + ([pad] if pad else [])
    n = sum(lens)
    s = n // c
    doc_start = np.repeat(np.cumsum([0] + lens[:-1]), lens)
    total = 0
    for t in range(c):
        busiest = 0
        for r in range(c):
            j = (r - t) % c
            qpos = np.arange(r * s, (r + 1) * s)
            first = np.maximum(doc_start[qpos], j * s)
            last = np.minimum(qpos, (j + 1) * s - 1)
            busiest = max(busiest, int(np.maximum(last - first + 1, 0).sum()))
        total += busiest
    return total


def _cost(docs, c):
    # the same cost form, written out independently for the oracle
    n = sum(docs)
    return 4e-8 * _critical(tuple(docs), c) + 1e-4 * n / c + 2e-6 * n + 0.05 * c + 0.1


def test_step_pairs_against_a_token_by_token_count():
    rng = np.random.default_rng(11)
    for _ in range(40):
        docs = [int(x) for x in rng.integers(1, 900, rng.integers(1, 7))]
        c = int(rng.choice([1, 2, 4, 8]))
        assert dcp.critical_pairs(docs, c) == _critical(tuple(docs), c), (docs, c)
    # one document over c ranks: P_crit is the last rank's work, (2c - 1) / c times the mean
    d = 64 * 8 * 16
    assert dcp.critical_pairs([d], 8) == (d // 8) ** 2 * 7 + (d // 8) * (d // 8 + 1) // 2
    # every rank's pairs over the ring add up to the micro-batch's pairs
    docs = [700, 1300, 250]
    per = dcp.step_pairs(docs, 4)
    assert per.sum() == sum(x * (x + 1) // 2 for x in dcp.ring_docs(docs, 4))


def test_fit_recovers_a_known_model():
    rng = np.random.default_rng(0)
    samples = []
    for tot in (8192, 16384, 32768, 65536):
        for dl in (256, 1024, 4096, 16384):
            if dl <= tot:
                for c in (1, 2, 4, 8):
                    docs = [dl] * (tot // dl)
                    samples.append((docs, c, MODEL.predict(docs, c) * (1 + 1e-4 * rng.standard_normal())))
    fit, err = dcp.fit_cost_model(samples)
    assert err < 1e-3
    for name in ("alpha", "beta", "eps", "gamma", "delta"):
        assert getattr(fit, name) == pytest.approx(getattr(MODEL, name), rel=2e-2)


def test_fit_keeps_every_cost_non_negative():
    # timings with no per-token term plus noise: an unconstrained fit may trade a negative
    # per-token cost against the others; every term is a cost, so the fit clamps it at zero
    rng = np.random.default_rng(0)   # with this noise an unconstrained fit gives eps < 0
    truth = dcp.CostModel(alpha=4e-8, beta=1e-4, eps=0.0, gamma=0.05, delta=0.1)
    samples = []
    for tot in (8192, 16384, 32768):
        for dl in (512, 2048, 8192):
            for c in (1, 2, 4, 8):
                docs = [dl] * (tot // dl)
                samples.append((docs, c, truth.predict(docs, c) * (1 + 0.05 * rng.standard_normal())))
    fit, _ = dcp.fit_cost_model(samples)
    assert min(fit.alpha, fit.beta, fit.eps, fit.gamma, fit.delta) >= 0.0
    assert fit.alpha == pytest.approx(truth.alpha, rel=0.2)


def test_cp_needed_is_the_smallest_power_of_two():
    assert [dcp.cp_needed(n, 1000, 8) for n in (1, 1000, 1001, 2000, 2001, 8000)] == [1, 1, 2, 2, 4, 8]
    with pytest.raises(ValueError):
        dcp.cp_needed(8001, 1000, 8)


@pytest.mark.parametrize("seed", range(6))
def test_plans_respect_every_constraint(seed):
    lengths = dcp.lognormal_lengths(seed, 200)
    for solve in (dcp.solve_dynamic, dcp.solve_static):
        plan = solve(lengths, 8, 16384, MODEL)
        dcp.check_plan(plan, lengths, 8, 16384)
        # the per-GPU loads are what the micro-batches charge
        loads = [0.0] * 8
        for mb in plan.micro_batches:
            t = MODEL.predict([lengths[i] for i in mb.seqs], mb.cp)
            for g in range(mb.group * mb.cp, (mb.group + 1) * mb.cp):
                loads[g] += t
        assert np.allclose(loads, plan.loads)


@pytest.mark.parametrize("seed", range(12))
def test_heuristic_near_the_exhaustive_optimum(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(3, 6))
    lengths = [int(x) for x in rng.integers(200, 4000, n)]
    opt = optimal_time(lengths, 4, 2048, _cost)
    got = dcp.solve_dynamic(lengths, 4, 2048, MODEL).time
    assert opt <= got + 1e-9                    # the oracle really is a lower bound
    assert got <= 1.5 * opt, (lengths, got, opt)


def test_oracle_on_a_hand_checked_case():
    # two sequences of 1500 tokens, 2 GPUs of 1000 tokens: each needs CP 2 and both share the
    # GPUs, so the best iteration runs them one after the other on both GPUs
    t = optimal_time([1500, 1500], 2, 1000, _cost)
    assert t == pytest.approx(2 * _cost([1500], 2))
    # one GPU of 4096 tokens: packing both into one micro-batch saves a fixed cost
    t = optimal_time([1000, 2000], 1, 4096, _cost)
    assert t == pytest.approx(_cost([1000, 2000], 1))


def test_dynamic_beats_static_packing_on_lognormal_batches():
    for seed in range(4):
        lengths = dcp.lognormal_lengths(seed, 256)
        dyn = dcp.solve_dynamic(lengths, 8, 16384, MODEL).time
        sta = dcp.solve_static(lengths, 8, 16384, MODEL).time
        assert dyn < sta
