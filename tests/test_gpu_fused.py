"""All-gather (fused multi-block) forward on the GPU: ringattn_fused_fwd against the fp64 oracle.

Every K/V block is resident and one launch computes the attention of a rank's
queries over all of them, so the result must equal full attention over the
union of the blocks.  Tolerances as for the bf16 ring: max |err| <= 1e-2 on O,
<= 1e-3 on LSE; rows that see no key have LSE = -inf and O = 0.
"""
import numpy as np
import pytest
import torch

import oracle
import ring_attention_ringattn_amd as ra
import synthetic
from tests.gpu_util import dev, max_abs, oracle_rows, print_case, thd_view

pytestmark = pytest.mark.gpu

TOL_O, TOL_L = 1e-2, 1e-3
BF = torch.bfloat16


def _fused(q, ks, vs, q_pos, kv_pos, mask, q_doc=None, kv_doc=None, put=None, flags=0):
    put = put or (lambda a: dev(a, BF))
    qd = put(q)
    out = torch.full(qd.shape, float("nan"), dtype=BF, device="cuda")
    if qd.stride() != out.stride():
        out = thd_view(out)
    lse = torch.full(qd.shape[:3], float("nan"), device="cuda")
    ra.ringattn_fused_fwd(qd, [put(k) for k in ks], [put(v) for v in vs], lse, out, dev(q_pos, torch.int32),
                          [dev(p, torch.int32) for p in kv_pos],
                          None if q_doc is None else dev(q_doc, torch.int32),
                          None if kv_doc is None else [dev(d, torch.int32) for d in kv_doc],
                          mask_mode={"none": ra.RA_MASK_NONE, "causal": ra.RA_MASK_CAUSAL,
                                     "doc_causal": ra.RA_MASK_DOC_CAUSAL}[mask], flags=flags)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def _check(out, lse, O, L):
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(lse), fin), "rows that see no key must have lse = -inf"
    e_o, e_l = max_abs(out, O), max_abs(lse[fin], L[fin])
    print(f"  max|dO| {e_o:.3g} max|dLSE| {e_l:.3g}", flush=True)
    assert e_o <= TOL_O and e_l <= TOL_L


def test_fused_zigzag_gqa_all_ranks():
    w = synthetic.WORKLOADS["c2"]
    print_case("fused: bf16, 32/8 GQA, D=128, S=8192, 4 zigzag shards, causal, every rank over all 4 blocks")
    inp = synthetic.make_inputs(w)
    pos = ra.sharding.shard_positions(w.seq, w.n_shards, w.sharding)
    O, L = oracle.attention_forward(inp["q"], inp["k"], inp["v"], np.arange(w.seq), np.arange(w.seq), "causal",
                                    row_block=256, skip_masked_columns=True)
    ks = [inp["k"][:, :, p] for p in pos]
    vs = [inp["v"][:, :, p] for p in pos]
    for r in range(w.n_shards):
        out, lse = _fused(inp["q"][:, :, pos[r]], ks, vs, pos[r], pos, "causal")
        _check(out, lse, O[:, :, pos[r]], L[:, :, pos[r]])


@pytest.mark.parametrize("rank", [0, 7])
def test_fused_full_size_rank_share_sampled_rows(rank):
    """All 8 blocks of a 131072-token zigzag context (16384 queries x 131072 keys) in one launch."""
    w = synthetic.WORKLOADS["c3"]
    print_case(f"fused: c3 rank {rank} of 8, 16384 queries over 8 resident blocks of 16384 keys")
    pos = ra.sharding.shard_positions(w.seq, w.n_shards, w.sharding)
    inp = synthetic.make_inputs(w, q_rows=pos[rank])
    out, lse = _fused(inp["q"], [inp["k"][:, :, p] for p in pos], [inp["v"][:, :, p] for p in pos], pos[rank], pos,
                      "causal")
    rng = np.random.default_rng(300 + rank)
    c = w.seq // (2 * w.n_shards)
    local = np.unique(np.concatenate([rng.choice(pos[rank].size, 40, replace=False), [0, c - 1, c, 2 * c - 1]]))
    O, L = oracle_rows(inp, pos[rank][local], "causal")
    _check(out[:, :, local], lse[:, :, local], O, L)


def test_fused_thd_doc_causal_all_ranks():
    print_case("fused: THD layout, doc-causal, 4 contiguous shards of a 4096-token packed stream")
    w = synthetic.small_workload("c5", seq=4096, n_shards=4, hq=4, hkv=2)
    inp = synthetic.make_inputs(w, backward=False)
    lens = synthetic.doc_lengths(11, 4096, median=300.0)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    doc = oracle.docs_from_cu_seqlens(cu, 4096)
    pos = ra.sharding.shard_positions(4096, 4, "contiguous")
    O, L = oracle.attention_forward(inp["q"], inp["k"], inp["v"], np.arange(4096), np.arange(4096), "doc_causal",
                                    doc, doc, skip_masked_columns=True)
    ks = [inp["k"][:, :, p] for p in pos]
    vs = [inp["v"][:, :, p] for p in pos]
    put = lambda a: thd_view(dev(a, BF))
    for r in range(4):
        out, lse = _fused(inp["q"][:, :, pos[r]], ks, vs, pos[r], pos, "doc_causal", doc[pos[r]],
                          [doc[p] for p in pos], put=put)
        _check(out, lse, O[:, :, pos[r]], L[:, :, pos[r]])


@pytest.mark.parametrize("case", [("none", 128, 3, 300, 333), ("causal", 128, 5, 200, 190),
                                  ("doc_causal", 64, 3, 257, 130), ("causal", 64, 16, 65, 70)],
                         ids=lambda c: "-".join(map(str, c)))
def test_fused_ragged_blocks(case):
    """Blocks with a ragged last tile, scattered positions and documents, up to the 16-block maximum."""
    mask, d, nb, sq, sk = case
    print_case(f"fused ragged {case}")
    rng = np.random.default_rng(sq * 100 + nb)
    rnd = lambda *s: synthetic.bf16_round(0.5 * rng.standard_normal(s).astype(np.float32))
    B, hq, hkv = 2, 4, 2
    q = rnd(B, hq, sq, d)
    ks = [rnd(B, hkv, sk, d) for _ in range(nb)]
    vs = [rnd(B, hkv, sk, d) for _ in range(nb)]
    perm = rng.permutation(sq + nb * sk).astype(np.int32)
    qp = perm[:sq]
    kps = [perm[sq + j * sk: sq + (j + 1) * sk] for j in range(nb)]
    docs = np.sort(rng.integers(0, 6, sq + nb * sk)).astype(np.int32)
    dm = mask == "doc_causal"
    out, lse = _fused(q, ks, vs, qp, kps, mask, docs[qp] if dm else None, [docs[p] for p in kps] if dm else None)
    kall = np.concatenate(kps)
    O, L = oracle.attention_forward(q, np.concatenate(ks, 2), np.concatenate(vs, 2), qp, kall, mask,
                                    docs[qp] if dm else None, docs[kall] if dm else None)
    _check(out, lse, O, L)


def test_fused_matches_ring_and_no_skip():
    """The same rank share through the 4-step ring and through one fused launch (with and without
    tile skipping) agree to the bf16 output rounding."""
    w = synthetic.small_workload("c2", seq=4096, n_shards=4, hq=8, hkv=2, seed=9)
    print_case("fused vs ring: 4096 tokens, 4 zigzag shards, rank 2")
    inp = synthetic.make_inputs(w)
    pos = ra.sharding.shard_positions(w.seq, 4, "zigzag")
    ks = [inp["k"][:, :, p] for p in pos]
    vs = [inp["v"][:, :, p] for p in pos]
    q = inp["q"][:, :, pos[2]]
    out_f, lse_f = _fused(q, ks, vs, pos[2], pos, "causal")
    out_n, lse_n = _fused(q, ks, vs, pos[2], pos, "causal", flags=ra.RA_NO_SKIP)
    qd = dev(q, BF)
    o_acc = torch.zeros(qd.shape, device="cuda")
    lse = torch.zeros(qd.shape[:3], device="cuda")
    out = torch.zeros_like(qd)
    for t in range(4):
        j = (2 - t) % 4
        ra.ringattn_step_fwd(qd, dev(ks[j], BF), dev(vs[j], BF), o_acc, lse, out, dev(pos[2], torch.int32),
                             dev(pos[j], torch.int32), flags=(ra.RA_STEP_FIRST if t == 0 else 0) |
                             (ra.RA_STEP_LAST if t == 3 else 0))
    torch.cuda.synchronize()
    assert max_abs(out_f, out.float().cpu().numpy()) <= 2 ** -7
    assert max_abs(lse_f, lse.cpu().numpy()) <= 1e-5
    assert max_abs(out_f, out_n) <= 2 ** -7 and max_abs(lse_f, lse_n) <= 1e-5


def test_run_driver_allgather_mode():
    """ringattn_run with RA_RUN_ALLGATHER: one fused launch per emulated rank over the home blocks."""
    w = synthetic.small_workload("c2", seq=4096, n_shards=4, hq=8, hkv=2, seed=21)
    print_case("run driver, all-gather mode: 4096 tokens, 4 zigzag shards, all ranks")
    inp = synthetic.make_inputs(w)
    pos = ra.sharding.shard_positions(w.seq, 4, "zigzag")
    O, L = oracle.attention_forward(inp["q"], inp["k"], inp["v"], np.arange(w.seq), np.arange(w.seq), "causal",
                                    skip_masked_columns=True)
    q = [dev(inp["q"][:, :, p], BF) for p in pos]
    kh = [dev(inp["k"][:, :, p], BF) for p in pos]
    vh = [dev(inp["v"][:, :, p], BF) for p in pos]
    out = [torch.full_like(x, float("nan")) for x in q]
    lse = [torch.full(x.shape[:3], float("nan"), device="cuda") for x in q]
    ra.ringattn_run(q, kh, vh, [dev(p, torch.int32) for p in pos], [dev(p, torch.int32) for p in pos], lse=lse,
                    out=out, flags=ra.RA_RUN_ALLGATHER)
    torch.cuda.synchronize()
    for r in range(4):
        _check(out[r].float().cpu().numpy(), lse[r].cpu().numpy(), O[:, :, pos[r]], L[:, :, pos[r]])
