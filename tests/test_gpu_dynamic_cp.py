"""Dynamic-CP's measuring path on the GPU: ring timing by the slowest rank, the cost-model fit
on a small grid, and a small plan executed."""
import numpy as np
import pytest

from ring_attention_ringattn_amd import dynamic_cp as dcp
from tests.gpu_util import print_case

pytestmark = pytest.mark.gpu


def test_ring_time_is_each_steps_slowest_rank():
    print_case("dynamic-cp: one 16384-token document over 4 contiguous ranks, 32/8 heads")
    t = dcp.time_micro_batch([16384], 4, reps=3)
    print(f"  ring {t.ms:.3f} ms, ranks {[round(x, 3) for x in t.per_rank_ms]}", flush=True)
    assert min(t.per_rank_ms) > 0
    assert t.ms >= max(t.per_rank_ms) - 1e-9          # a ring is never faster than its slowest rank
    # causal document split contiguously: rank r's queries see r + 1/2 blocks of keys
    assert int(np.argmax(t.per_rank_ms)) == 3 and int(np.argmin(t.per_rank_ms)) == 0
    assert t.ms >= 1.3 * sum(t.per_rank_ms) / 4     # (2c - 1)/c = 1.75 times the mean rank, less launch costs


def test_fit_and_plan_on_a_small_grid():
    print_case("dynamic-cp: fit on 12 micro-batches (4/2 heads), plan and execute 10 sequences on 4 GPUs")
    timing = dict(hq=4, hkv=2, reps=2)
    samples = dcp.measure(grid_tokens=(4096, 8192), doc_lengths=(512, 4096), cps=(1, 2, 4), **timing)
    assert len(samples) == 12 and all(ms > 0 for _, _, ms in samples)
    model, err = dcp.fit_cost_model(samples)
    print(f"  fit: {model}, worst relative error {err:.3f}", flush=True)
    assert np.isfinite(err) and err < 1.0
    lengths = dcp.lognormal_lengths(3, 10, median=1024, hi=8192)
    plan = dcp.solve_dynamic(lengths, 4, 8192, model)
    dcp.check_plan(plan, lengths, 4, 8192)
    t = dcp.execute(plan, lengths, 4, **timing)
    print(f"  plan of {len(plan.micro_batches)} micro-batches: predicted {plan.time:.3f} ms, measured {t:.3f} ms",
          flush=True)
    assert t > 0 and np.isfinite(t)
