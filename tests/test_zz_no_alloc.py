"""The allocation-free forward step (ringattn_step_fwd_noalloc) against ringattn_step_fwd.

Both run the same kernels on the same inputs, so their outputs must agree bit for bit; the
final results are also checked against the fp64 oracle (bf16 bounds: O 1e-2, LSE 1e-3).
Three calls in a row share the library's one scratch array: a 16384 x 16384 diagonal step
(the largest block the scratch holds at 8 kv heads, D = 128), then two smaller ragged steps,
so the later calls run over what the first left in the array.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import ring_attention_ringattn_amd as ra
import synthetic
from tests.gpu_util import dev, max_abs, print_case

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _both(q, k, v, qp, kp, qd, kd, mask, flags, state):
    """Run the step through both entry points; `state` holds each path's (o_acc, lse, out)."""
    for name, fn in (("ws", ra.ringattn_step_fwd), ("noalloc", ra.ringattn_step_fwd_noalloc)):
        o, l, out = state[name]
        fn(q, k, v, o, l, out, qp, kp, qd, kd, mask_mode=mask, flags=flags)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16 if t.dtype == BF else torch.int32)   # NaN fill compares equal too
    for a, b in zip(state["ws"], state["noalloc"]):
        assert torch.equal(bits(a), bits(b)), "the allocation-free step must reproduce ringattn_step_fwd bit for bit"


def _state(B, hq, sq, d):
    mk = lambda: (torch.full((B, hq, sq, d), 3.0, device="cuda"), torch.full((B, hq, sq), 3.0, device="cuda"),
                  torch.full((B, hq, sq, d), float("nan"), dtype=BF, device="cuda"))
    return {"ws": mk(), "noalloc": mk()}


def test_noalloc_step_matches_workspace_step_twice():
    # 1) a 16384-token query shard against its own 16384-key block (diagonal: partial tiles), 32/8 heads
    print_case("noalloc: 16384 x 16384 diagonal step, 32/8 heads, D=128, causal")
    w = synthetic.small_workload("c3", seq=32768, n_shards=2, seed=77)
    pos = ra.sharding.shard_positions(w.seq, 2, "zigzag")
    inp = synthetic.make_inputs(w, q_rows=pos[0])
    k, v = inp["k"][:, :, pos[0]], inp["v"][:, :, pos[0]]
    qp = dev(pos[0], torch.int32)
    st = _state(1, 32, 16384, 128)
    _both(dev(inp["q"], BF), dev(k, BF), dev(v, BF), qp, qp, None, None, ra.RA_MASK_CAUSAL,
          ra.RA_STEP_FIRST | ra.RA_STEP_LAST, st)
    rows = np.unique(np.concatenate([np.random.default_rng(1).choice(16384, 40, replace=False),
                                     [0, 63, 64, 8191, 8192, 16383]]))
    O, L = oracle.attention_forward(inp["q"][:, :, rows], k, v, pos[0][rows], pos[0], "causal", row_block=128,
                                    skip_masked_columns=True)
    o, l, out = st["noalloc"]
    assert max_abs(out[:, :, rows].float().cpu().numpy(), O) <= 1e-2
    assert max_abs(o[:, :, rows].cpu().numpy(), O) <= 1e-2
    assert max_abs(l[:, :, rows].cpu().numpy(), L) <= 1e-3

    # 2) a smaller ragged problem, two steps (FIRST, then LAST), D = 64, document-causal
    print_case("noalloc: then two ragged doc-causal steps, 4/2 heads, D=64, 300 queries, 2 x 1100 keys")
    rng = np.random.default_rng(zlib.crc32(b"noalloc"))
    rnd = lambda *s: synthetic.bf16_round(0.5 * rng.standard_normal(s).astype(np.float32))
    sq, sk, d = 300, 1100, 64
    q, k1, v1, k2, v2 = rnd(1, 4, sq, d), rnd(1, 2, sk, d), rnd(1, 2, sk, d), rnd(1, 2, sk, d), rnd(1, 2, sk, d)
    perm = rng.permutation(sq + 2 * sk).astype(np.int32)
    qpos, kp1, kp2 = perm[:sq], perm[sq:sq + sk], perm[sq + sk:]
    docs = np.sort(rng.integers(0, 5, sq + 2 * sk)).astype(np.int32)
    st = _state(1, 4, sq, d)
    for flags, kk, vv, kp in ((ra.RA_STEP_FIRST, k1, v1, kp1), (ra.RA_STEP_LAST, k2, v2, kp2)):
        _both(dev(q, BF), dev(kk, BF), dev(vv, BF), dev(qpos, torch.int32), dev(kp, torch.int32),
              dev(docs[qpos], torch.int32), dev(docs[kp], torch.int32), ra.RA_MASK_DOC_CAUSAL, flags, st)
    O, L = oracle.attention_forward(q, np.concatenate([k1, k2], 2), np.concatenate([v1, v2], 2), qpos,
                                    np.concatenate([kp1, kp2]), "doc_causal", docs[qpos],
                                    docs[np.concatenate([kp1, kp2])])
    o, l, out = st["noalloc"]
    fin = np.isfinite(L)
    got_l = l.cpu().numpy()
    assert np.array_equal(np.isfinite(got_l), fin)
    assert max_abs(got_l[fin], L[fin]) <= 1e-3
    assert max_abs(o.cpu().numpy(), O) <= 1e-2 and max_abs(out.float().cpu().numpy(), O) <= 1e-2


def test_noalloc_rejects_a_block_too_large_for_its_scratch():
    print_case("noalloc: 32768-key block of 8 kv heads is refused, outputs untouched")
    q = torch.zeros(1, 8, 128, 128, dtype=BF, device="cuda")
    k = torch.zeros(1, 8, 32768, 128, dtype=BF, device="cuda")
    o = torch.full((1, 8, 128, 128), 3.0, device="cuda")
    l = torch.full((1, 8, 128), 3.0, device="cuda")
    p = torch.arange(32768, dtype=torch.int32, device="cuda")
    with pytest.raises(ra.RingAttnError) as e:
        ra.ringattn_step_fwd_noalloc(q, k, k, o, l, None, p[:128], p)
    assert e.value.status == ra._lib.RA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(o == 3.0) and torch.all(l == 3.0)
