"""Backward parity on the GPU: ringattn_run(pass=backward) against the fp64 oracle.

Tolerance: dQ, dK, dV relative L2 error <= 2e-2 (bf16 inputs).  dK/dV of a
block collect the contributions of the emulated ranks' queries only, which is
what the oracle computes when given just those query rows.
"""
import numpy as np
import pytest
import torch

import oracle
import ring_attention_ringattn_amd as ra
import synthetic
from tests.gpu_util import Ring, dev, max_abs, print_case, rel_l2

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _global_grads(inp, rows, mask, doc=None):
    """Oracle dQ (for `rows`) and dK, dV (contributions of `rows`) over the whole context."""
    s = inp["k"].shape[2]
    where = {int(g): i for i, g in enumerate(inp["q_rows"])}
    sel = [where[int(g)] for g in rows]
    return oracle.attention_backward(inp["q"][:, :, sel], inp["k"], inp["v"], inp["do"][:, :, sel], rows,
                                     np.arange(s), mask, None if doc is None else doc[rows], doc,
                                     row_block=128, skip_masked_columns=mask != "none")


def _check(ring, inp, mask, doc=None, rows_per_rank=None):
    rows = np.concatenate([ring.pos[r] for r in ring.ranks])
    dQ, dK, dV = _global_grads(inp, rows, mask, doc)
    off = 0
    for i, r in enumerate(ring.ranks):
        n = ring.pos[r].size
        e = rel_l2(ring.numpy("dq")[i], dQ[:, :, off:off + n])
        print(f"  rank {r}: dQ rel L2 {e:.3g}", flush=True)
        assert e <= TOL
        off += n
    for n_, p in enumerate(ring.pos):
        ek = rel_l2(ring.numpy("dk")[n_], dK[:, :, p])
        ev = rel_l2(ring.numpy("dv")[n_], dV[:, :, p])
        print(f"  block {n_}: dK rel L2 {ek:.3g} dV rel L2 {ev:.3g}", flush=True)
        assert ek <= TOL and ev <= TOL


def test_bwd_zigzag_ring_all_ranks():
    print_case("bwd: zigzag 4 ranks, 2048 tokens, 8/2 GQA heads, D=128, all ranks")
    w = synthetic.small_workload("c4", seq=2048, n_shards=4, hq=8, hkv=2, seed=41)
    inp = synthetic.make_inputs(w)
    pos = ra.sharding.shard_positions(w.seq, 4, "zigzag")
    ring = Ring(inp["q"], inp["k"], inp["v"], pos, "causal", "bf16", range(4), do_glob=inp["do"])
    ring.forward().backward()
    _check(ring, inp, "causal")
    # the other staging modes give the same bits: serial copies, DMA-engine copies, poisoned slots
    ref = [[t.clone() for t in getattr(ring, n)] for n in ("dq", "dk", "dv")]
    for flags, cs in ((ra.RA_RUN_SERIAL_COPY, "side"), (ra.RA_RUN_COPY_ENGINE, "side"),
                      (ra.RA_RUN_COPY_ENGINE | ra.RA_RUN_POISON, "side"), (ra.RA_RUN_POISON, "side")):
        print(f"  backward flags {flags}", flush=True)
        ring.backward(flags=flags, copy_stream=cs)
        for n, r in zip(("dq", "dk", "dv"), ref):
            for x, y in zip(getattr(ring, n), r):
                assert torch.equal(x, y), (flags, n)


def test_bwd_rank_share_medium():
    """The launch configuration of the 262144-token share, scaled to 16384 tokens: rank 0 of 8, 32/8 heads."""
    print_case("bwd: rank 0 of 8 zigzag shards, 16384 tokens, 32/8 GQA heads, D=128")
    w = synthetic.small_workload("c4", seq=16384, seed=42)
    pos = ra.sharding.shard_positions(w.seq, 8, "zigzag")
    inp = synthetic.make_inputs(w, q_rows=pos[0])
    ring = Ring(None, inp["k"], inp["v"], pos, "causal", "bf16", [0], q_shards=[inp["q"]], do_shards=[inp["do"]])
    ring.forward().backward()
    _check(ring, inp, "causal")


def test_bwd_causal_multi_chunk_work_list():
    """Causal dK/dV workgroups whose work list (query head x 64-row tile) spans several chunks:
    rank 0 of a 16384-token context over 2 zigzag shards, 4 query heads on 1 kv head, so each
    key workgroup walks 4 x 128 = 512 items.  Every dQ, dK, dV element against the oracle."""
    print_case("bwd: rank 0 of 2 zigzag shards, 16384 tokens, 4/1 heads, D=128 (512 work items per key tile)")
    w = synthetic.small_workload("c4", seq=16384, n_shards=2, hq=4, hkv=1, seed=44)
    pos = ra.sharding.shard_positions(w.seq, 2, "zigzag")
    inp = synthetic.make_inputs(w, q_rows=pos[0])
    ring = Ring(None, inp["k"], inp["v"], pos, "causal", "bf16", [0], q_shards=[inp["q"]], do_shards=[inp["do"]])
    ring.forward().backward()
    _check(ring, inp, "causal")


def test_bwd_fp32_contiguous_ring_all_ranks():
    """fp32 backward at the fp32 workload's shape (2 heads, D = 64, 512 tokens over 4 contiguous
    shards, causal, all ranks): dQ, dK, dV max |err| <= 1e-5, the fp32 bound."""
    print_case("bwd fp32: 4 contiguous ranks, 512 tokens, 2 heads, D=64, causal")
    w = synthetic.small_workload("c1", backward=True)
    inp = synthetic.make_inputs(w)
    pos = ra.sharding.shard_positions(w.seq, w.n_shards, w.sharding)
    ring = Ring(inp["q"], inp["k"], inp["v"], pos, "causal", "f32", range(4), do_glob=inp["do"])
    ring.forward().backward()
    s_all = np.arange(w.seq)
    dQ, dK, dV = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], s_all, s_all, "causal")
    for i, r in enumerate(ring.ranks):
        e = max_abs(ring.numpy("dq")[i], dQ[:, :, pos[r]])
        print(f"  rank {r}: dQ max abs {e:.3g}", flush=True)
        assert e <= 1e-5
    for n_, p in enumerate(pos):
        ek, ev = max_abs(ring.numpy("dk")[n_], dK[:, :, p]), max_abs(ring.numpy("dv")[n_], dV[:, :, p])
        print(f"  block {n_}: dK max abs {ek:.3g} dV max abs {ev:.3g}", flush=True)
        assert ek <= 1e-5 and ev <= 1e-5


@pytest.mark.parametrize("case", [("causal", 64, 1, 2, 1, 100, 150), ("none", 128, 2, 2, 2, 65, 70),
                                  ("doc_causal", 64, 1, 4, 2, 130, 200), ("causal", 128, 1, 3, 1, 257, 190)],
                         ids=lambda c: "-".join(map(str, c)))
def test_step_bwd_fp32_ragged(case):
    """fp32 backward step on ragged sizes with scattered positions and documents: max |err| <= 1e-5."""
    mask, d, B, hq, hkv, sq, sk = case
    print_case(f"step_bwd fp32 {case}")
    rng = np.random.default_rng(sq * 7 + sk)
    rnd = lambda *sh: rng.standard_normal(sh).astype(np.float32)
    q, k, v, do = rnd(B, hq, sq, d), rnd(B, hkv, sk, d), rnd(B, hkv, sk, d), rnd(B, hq, sq, d)
    perm = rng.permutation(sq + sk).astype(np.int32)
    qp, kp = perm[:sq], perm[sq:]
    docs = np.sort(rng.integers(0, 4, sq + sk)).astype(np.int32)
    qd, kd = (docs[qp], docs[kp]) if mask == "doc_causal" else (None, None)
    O, L = oracle.attention_forward(q, k, v, qp, kp, mask, qd, kd)
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, qp, kp, mask, qd, kd)
    out = dev(O)
    delta = torch.zeros(B, hq, sq, device="cuda")
    ra.ringattn_bwd_preprocess(out, dev(do), delta)
    dq = torch.zeros(B, hq, sq, d, device="cuda")
    dk = torch.zeros(B, hkv, sk, d, device="cuda")
    dv = torch.zeros(B, hkv, sk, d, device="cuda")
    doc_t = (lambda x: None if x is None else dev(x, torch.int32))
    ra.ringattn_step_bwd(dev(q), dev(k), dev(v), dev(do), dev(L), delta, dq, dk, dv, dev(qp, torch.int32),
                         dev(kp, torch.int32), doc_t(qd), doc_t(kd),
                         mask_mode={"none": ra.RA_MASK_NONE, "causal": ra.RA_MASK_CAUSAL,
                                    "doc_causal": ra.RA_MASK_DOC_CAUSAL}[mask])
    torch.cuda.synchronize()
    for got, ref, name in ((dq, dQ, "dQ"), (dk, dK, "dK"), (dv, dV, "dV")):
        e = max_abs(got.cpu().numpy(), ref)
        print(f"  {name} max abs {e:.3g}", flush=True)
        assert e <= 1e-5


def test_bwd_doc_causal_thd_all_ranks():
    print_case("bwd: packed documents, THD layout, 4 contiguous shards of 8192 tokens, 8/2 heads")
    w = synthetic.small_workload("c5", seq=8192, n_shards=4, hq=8, hkv=2, seed=43)
    inp = synthetic.make_inputs(w)
    lens = synthetic.doc_lengths(43, 8192, median=600.0)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    doc = oracle.docs_from_cu_seqlens(cu, 8192)
    pos = ra.sharding.shard_positions(8192, 4, "contiguous")
    ring = Ring(inp["q"], inp["k"], inp["v"], pos, "doc_causal", "bf16", range(4), doc=doc, layout="thd",
                do_glob=inp["do"])
    ring.forward().backward()
    _check(ring, inp, "doc_causal", doc)


@pytest.mark.parametrize("case", [("none", 64, 130, 200), ("causal", 64, 257, 190), ("causal", 128, 100, 333),
                                  # odd GQA group sizes (MHA, 3 heads per kv head): one query head per dQ workgroup
                                  ("none", 64, 130, 200, 2, 2), ("causal", 128, 100, 333, 3, 1)],
                         ids=lambda c: "-".join(map(str, c)))
def test_step_bwd_ragged(case):
    """One backward step on ragged sizes with scattered positions (step entry point, D=64 and 128)."""
    mask, d, sq, sk, *heads = case
    print_case(f"step_bwd {case}")
    rng = np.random.default_rng(sq * 1000 + sk)
    rnd = lambda *s: synthetic.bf16_round(0.5 * rng.standard_normal(s).astype(np.float32))
    B, (hq, hkv) = 2, (heads or (4, 2))
    q, k, v, do = rnd(B, hq, sq, d), rnd(B, hkv, sk, d), rnd(B, hkv, sk, d), rnd(B, hq, sq, d)
    perm = rng.permutation(sq + sk).astype(np.int32)
    qp, kp = perm[:sq], perm[sq:]
    if mask == "causal":
        qp = np.maximum(qp, 5).astype(np.int32)     # every query sees at least one key below it
        kp[0] = 0
    O, L = oracle.attention_forward(q, k, v, qp, kp, mask)
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, qp, kp, mask)
    bf = torch.bfloat16
    out = dev(O, bf)
    delta = torch.zeros(B, hq, sq, device="cuda")
    ra.ringattn_bwd_preprocess(out, dev(do, bf), delta)
    dq = torch.zeros(B, hq, sq, d, device="cuda")
    dk = torch.zeros(B, hkv, sk, d, device="cuda")
    dv = torch.zeros(B, hkv, sk, d, device="cuda")
    ra.ringattn_step_bwd(dev(q, bf), dev(k, bf), dev(v, bf), dev(do, bf), dev(L), delta, dq, dk, dv,
                         dev(qp, torch.int32), dev(kp, torch.int32),
                         mask_mode={"none": ra.RA_MASK_NONE, "causal": ra.RA_MASK_CAUSAL}[mask])
    torch.cuda.synchronize()
    ref_delta = np.sum(do.astype(np.float64) * out.float().cpu().numpy(), axis=-1)
    assert max_abs(delta.cpu().numpy(), ref_delta) <= 1e-4
    for got, ref, name in ((dq, dQ, "dQ"), (dk, dK, "dK"), (dv, dV, "dV")):
        e = rel_l2(got.cpu().numpy(), ref)
        print(f"  {name} rel L2 {e:.3g}", flush=True)
        assert e <= TOL


def test_bwd_full_size_rank_share():
    """262144-token context, rank 0 of 8 (32768 queries, 8 blocks of 32768 keys), forward + backward.

    Exact per sampled row: O, LSE and dQ.  For dK/dV the identities that hold
    at any size: summed over every key of every block, dK vanishes (each row's
    dS sums to zero) and dV equals the sum of the rank's dO rows over the GQA
    group (each row's weights sum to one).
    """
    w = synthetic.WORKLOADS["c4"]
    print_case("c4: bf16 rank 0 of 8, 32768 local queries, 8 steps of 32768 keys, forward + backward")
    pos = ra.sharding.shard_positions(w.seq, w.n_shards, w.sharding)
    inp = synthetic.make_inputs(w, q_rows=pos[0])
    ring = Ring(None, inp["k"], inp["v"], pos, "causal", "bf16", [0], q_shards=[inp["q"]], do_shards=[inp["do"]])
    ring.forward().backward()
    rng = np.random.default_rng(7)
    c = w.seq // (2 * w.n_shards)
    local = np.unique(np.concatenate([rng.choice(pos[0].size, 24, replace=False), [0, c - 1, c, 2 * c - 1]]))
    rows = pos[0][local]
    O, L = oracle.attention_forward(inp["q"][:, :, local], inp["k"], inp["v"], rows, np.arange(w.seq), "causal",
                                    row_block=128, skip_masked_columns=True)
    assert max_abs(ring.numpy("out")[0][:, :, local], O) <= 1e-2
    assert max_abs(ring.numpy("lse")[0][:, :, local], L) <= 1e-3
    dQ, _, _ = oracle.attention_backward(inp["q"][:, :, local], inp["k"], inp["v"], inp["do"][:, :, local], rows,
                                         np.arange(w.seq), "causal", row_block=128, skip_masked_columns=True)
    e = rel_l2(ring.numpy("dq")[0][:, :, local], dQ)
    print(f"  sampled dQ rows rel L2 {e:.3g}", flush=True)
    assert e <= TOL
    dk_sum = sum(t.double().sum(dim=2) for t in ring.dk)           # [B, Hkv, D]
    dk_norm = torch.sqrt(sum((t.double() ** 2).sum(dim=2) for t in ring.dk))
    ratio = float((dk_sum.norm() / dk_norm.norm()).item())
    print(f"  |sum_j dK_j| / sqrt(sum_j |dK_j|^2) = {ratio:.3g}", flush=True)
    assert ratio <= 5e-2
    dv_sum = sum(t.double().sum(dim=2) for t in ring.dv).cpu().numpy()
    do_sum = inp["do"].astype(np.float64).reshape(1, w.hkv, w.hq // w.hkv, -1, w.head_dim).sum(axis=(2, 3))
    e = rel_l2(dv_sum, do_sum)
    print(f"  sum_j dV_j vs group sum of dO: rel L2 {e:.3g}", flush=True)
    assert e <= TOL
    for t in ring.dq + ring.dk + ring.dv:
        assert torch.isfinite(t).all()

    # Element-wise dK/dV at full size: the same launch configuration again, with dO kept on a
    # sample of rows of GQA group 0 (query heads 0-3) -- one random row of every 64-row query
    # tile plus the chunk edges -- and zero everywhere else.  A row with dO = 0 has dP = 0 and
    # delta = 0, so it adds exactly nothing to dQ, dK or dV; the oracle given only the sampled
    # rows is then exact for every key of every block.  Other kv heads must stay exactly zero.
    g = w.hq // w.hkv
    tiles = pos[0].size // 64
    local = np.unique(np.concatenate([np.arange(tiles) * 64 + rng.integers(0, 64, tiles), [0, c - 1, c, 2 * c - 1]]))
    sparse = np.zeros_like(inp["do"])
    sparse[:, :g, local] = inp["do"][:, :g, local]
    ring.do = [dev(sparse, torch.bfloat16)]
    print_case(f"c4 sparse dO: {local.size} rows of query heads 0-{g - 1}, backward again")
    ring.backward()
    _, dK, dV = oracle.attention_backward(inp["q"][:, :g, local], inp["k"][:, :1], inp["v"][:, :1],
                                          inp["do"][:, :g, local], pos[0][local], np.arange(w.seq), "causal",
                                          row_block=128, skip_masked_columns=True)
    head0 = lambda t: t[:, :1].double().cpu().numpy()
    for n_, p in enumerate(pos):
        ek, ev = rel_l2(head0(ring.dk[n_]), dK[:, :, p]), rel_l2(head0(ring.dv[n_]), dV[:, :, p])
        print(f"  block {n_}, kv head 0: dK rel L2 {ek:.3g} dV rel L2 {ev:.3g}", flush=True)
        assert ek <= TOL and ev <= TOL
        assert not ring.dk[n_][:, 1:].any() and not ring.dv[n_][:, 1:].any(), "kv heads without dO must stay zero"
    others = torch.from_numpy(np.setdiff1d(np.arange(pos[0].size), local)).cuda()
    dq = ring.dq[0]
    assert not dq[:, g:].any() and not dq[:, :g].index_select(2, others).any(), "rows without dO must have dQ = 0"


def test_c5_full_size_packed_documents():
    """65536 packed tokens of lognormal documents (seed 5: 22 documents), document-causal mask,
    4 contiguous shards, all ranks, 32/8 heads, forward + backward: the benchmark's packed
    configuration, with the document ids made on the device from cu_seqlens as the benchmark does.

    Exact per sampled row: O, LSE and dQ (random rows, the first and last row of every document
    and the rows next to each shard boundary).  Exact per document: dK and dV of every key of two
    whole documents -- the shortest one and the one that straddles the first shard boundary --
    from the oracle given that document's query rows (no other row sees its keys).
    """
    w = synthetic.WORKLOADS["c5"]
    print_case("c5: 65536 packed tokens, 22 documents, doc-causal, 4 contiguous shards, 32/8 heads, fwd + bwd")
    inp = synthetic.make_inputs(w)
    cu = inp["cu_seqlens"]
    doc = oracle.docs_from_cu_seqlens(cu, w.seq)
    n, S = w.n_shards, w.shard_len
    pos = ra.sharding.shard_positions(w.seq, n, w.sharding)
    ring = Ring(inp["q"], inp["k"], inp["v"], pos, "doc_causal", "bf16", range(n), doc=doc, do_glob=inp["do"])
    tcu = dev(cu, torch.int32)
    ring.q_doc = [ra.ringattn_docs_from_cu_seqlens(tcu, int(pos[r][0]), pos[r].size) for r in ring.ranks]
    ring.kv_doc = [ra.ringattn_docs_from_cu_seqlens(tcu, int(p[0]), p.size) for p in pos]
    ring.forward().backward()
    for i in range(n):
        assert np.array_equal(ring.q_doc[i].cpu().numpy(), doc[pos[i]])
    out, lse, dq = (np.concatenate(ring.numpy(x), axis=2) for x in ("out", "lse", "dq"))
    dk, dv = (np.concatenate(ring.numpy(x), axis=2) for x in ("dk", "dv"))   # contiguous: global order
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))

    rng = np.random.default_rng(5)
    bounds = np.concatenate([cu[:-1], cu[1:] - 1, np.arange(1, n) * S - 1, np.arange(1, n) * S])
    rows = np.unique(np.concatenate([rng.choice(w.seq, 24, replace=False), bounds]))
    args = dict(row_block=128, skip_masked_columns=True)
    kpos = np.arange(w.seq)
    O, L = oracle.attention_forward(inp["q"][:, :, rows], inp["k"], inp["v"], rows, kpos, "doc_causal",
                                    doc[rows], doc, **args)
    print(f"  {rows.size} sampled rows: O max abs {max_abs(out[:, :, rows], O):.3g}, "
          f"LSE max abs {max_abs(lse[:, :, rows], L):.3g}", flush=True)
    assert max_abs(out[:, :, rows], O) <= 1e-2
    assert max_abs(lse[:, :, rows], L) <= 1e-3
    dQ, _, _ = oracle.attention_backward(inp["q"][:, :, rows], inp["k"], inp["v"], inp["do"][:, :, rows], rows, kpos,
                                         "doc_causal", doc[rows], doc, **args)
    e = rel_l2(dq[:, :, rows], dQ)
    print(f"  sampled dQ rows rel L2 {e:.3g}", flush=True)
    assert e <= TOL

    lens = np.diff(cu)
    straddle = int(doc[S])   # the document holding the first token of shard 1
    assert doc[S - 1] == straddle, "the seed-5 stream has a document across the first shard boundary"
    for d in sorted({int(np.argmin(lens)), straddle}):
        r = np.arange(cu[d], cu[d + 1])
        _, dK, dV = oracle.attention_backward(inp["q"][:, :, r], inp["k"], inp["v"], inp["do"][:, :, r], r, kpos,
                                              "doc_causal", doc[r], doc, **args)
        ek, ev = rel_l2(dk[:, :, r], dK[:, :, r]), rel_l2(dv[:, :, r], dV[:, :, r])
        print(f"  document {d} ({r.size} tokens, keys {r[0]}..{r[-1]}): dK rel L2 {ek:.3g}, dV rel L2 {ev:.3g}",
              flush=True)
        assert ek <= TOL and ev <= TOL


def test_step_fwd_bwd_largest_block():
    """A key/value block of RA_MAX_SK = 262144 keys (4096 tiles: the largest tile index a work-list
    entry holds), 130 sorted query positions spread over the block (a query near the end sees every
    tile), causal, 2/1 heads, D = 128: forward (one step, first and last) and backward, every output
    against the oracle."""
    sk, sq, d, hq, hkv = ra.RA_MAX_SK, 130, 128, 2, 1
    print_case(f"step fwd+bwd bf16, sk = RA_MAX_SK = {sk}, sq = {sq}, causal, {hq}/{hkv} heads, D={d}")
    rng = np.random.default_rng(2718)
    rnd = lambda *s: synthetic.bf16_round(0.5 * rng.standard_normal(s).astype(np.float32))
    q, k, v, do = rnd(1, hq, sq, d), rnd(1, hkv, sk, d), rnd(1, hkv, sk, d), rnd(1, hq, sq, d)
    kp = np.arange(sk, dtype=np.int32)
    edges = [0, 63, 64, sk - 65, sk - 64, sk - 1]
    rest = rng.choice(np.setdiff1d(np.arange(sk), edges), sq - len(edges), replace=False)
    qp = np.sort(np.concatenate([edges, rest])).astype(np.int32)
    O, L = oracle.attention_forward(q, k, v, qp, kp, "causal", skip_masked_columns=True)
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, qp, kp, "causal", row_block=32, skip_masked_columns=True)
    bf = torch.bfloat16
    o_acc = torch.zeros(1, hq, sq, d, device="cuda")
    lse = torch.zeros(1, hq, sq, device="cuda")
    out = torch.full((1, hq, sq, d), float("nan"), dtype=bf, device="cuda")
    qd, kd, vd = dev(q, bf), dev(k, bf), dev(v, bf)
    qpd, kpd = dev(qp, torch.int32), dev(kp, torch.int32)
    ra.ringattn_step_fwd(qd, kd, vd, o_acc, lse, out, qpd, kpd, None, None, mask_mode=ra.RA_MASK_CAUSAL,
                         flags=ra.RA_STEP_FIRST | ra.RA_STEP_LAST)
    torch.cuda.synchronize()
    eo, el = max_abs(out.float().cpu().numpy(), O), max_abs(lse.cpu().numpy(), L)
    print(f"  forward: O max abs {eo:.3g}, LSE max abs {el:.3g}", flush=True)
    assert eo <= 1e-2 and el <= 1e-3
    delta = torch.zeros(1, hq, sq, device="cuda")
    ra.ringattn_bwd_preprocess(out, dev(do, bf), delta)
    dq = torch.zeros(1, hq, sq, d, device="cuda")
    dk = torch.zeros(1, hkv, sk, d, device="cuda")
    dv = torch.zeros(1, hkv, sk, d, device="cuda")
    ra.ringattn_step_bwd(qd, kd, vd, dev(do, bf), lse, delta, dq, dk, dv, qpd, kpd, mask_mode=ra.RA_MASK_CAUSAL)
    torch.cuda.synchronize()
    for got, ref, name in ((dq, dQ, "dQ"), (dk, dK, "dK"), (dv, dV, "dV")):
        e = rel_l2(got.cpu().numpy(), ref)
        print(f"  {name} rel L2 {e:.3g}", flush=True)
        assert e <= TOL


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_fwd_bwd_explicit_scale_and_no_skip(dtype):
    """A softmax scale other than 1/sqrt(D) (0.3), forward and backward against the oracle at that
    scale; the backward again with tile skipping off gives the same bits (fully masked tiles add
    exact zeros)."""
    d, B, hq, hkv, sq, sk, scale = 128, 1, 4, 2, 190, 333, 0.3
    print_case(f"step fwd+bwd {dtype}, softmax_scale {scale}, causal, D={d}, sq={sq}, sk={sk}; bwd with RA_NO_SKIP")
    rng = np.random.default_rng(31415)
    wdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rnd = (lambda *s: synthetic.bf16_round(0.5 * rng.standard_normal(s).astype(np.float32))) if dtype == "bf16" \
        else (lambda *s: rng.standard_normal(s).astype(np.float32))
    q, k, v, do = rnd(B, hq, sq, d), rnd(B, hkv, sk, d), rnd(B, hkv, sk, d), rnd(B, hq, sq, d)
    perm = rng.permutation(sq + sk).astype(np.int32)
    qp, kp = np.maximum(perm[:sq], 5).astype(np.int32), perm[sq:]
    kp[0] = 0
    O, L = oracle.attention_forward(q, k, v, qp, kp, "causal", scale=scale)
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, qp, kp, "causal", scale=scale)
    o_acc = torch.zeros(B, hq, sq, d, device="cuda")
    lse = torch.zeros(B, hq, sq, device="cuda")
    out = torch.full((B, hq, sq, d), float("nan"), dtype=wdt, device="cuda")
    qd, kd, vd, dod = dev(q, wdt), dev(k, wdt), dev(v, wdt), dev(do, wdt)
    qpd, kpd = dev(qp, torch.int32), dev(kp, torch.int32)
    ra.ringattn_step_fwd(qd, kd, vd, o_acc, lse, out, qpd, kpd, mask_mode=ra.RA_MASK_CAUSAL,
                         flags=ra.RA_STEP_FIRST | ra.RA_STEP_LAST, softmax_scale=scale)
    torch.cuda.synchronize()
    tol_o, tol_l = (1e-2, 1e-3) if dtype == "bf16" else (1e-5, 1e-5)
    eo, el = max_abs(out.float().cpu().numpy(), O), max_abs(lse.cpu().numpy(), L)
    print(f"  forward: O max abs {eo:.3g}, LSE max abs {el:.3g}", flush=True)
    assert eo <= tol_o and el <= tol_l
    # the backward from the oracle's O and LSE (as the other step tests), so it is checked on its own
    delta = torch.zeros(B, hq, sq, device="cuda")
    ra.ringattn_bwd_preprocess(dev(O, wdt), dod, delta)
    lse_ref = dev(L)
    grads = []
    for flags in (0, ra.RA_NO_SKIP):
        dq = torch.zeros(B, hq, sq, d, device="cuda")
        dk = torch.zeros(B, hkv, sk, d, device="cuda")
        dv = torch.zeros(B, hkv, sk, d, device="cuda")
        ra.ringattn_step_bwd(qd, kd, vd, dod, lse_ref, delta, dq, dk, dv, qpd, kpd, mask_mode=ra.RA_MASK_CAUSAL,
                             flags=flags, softmax_scale=scale)
        torch.cuda.synchronize()
        grads.append((dq, dk, dv))
    for got, ref, name in zip(grads[0], (dQ, dK, dV), ("dQ", "dK", "dV")):
        if dtype == "bf16":
            e = rel_l2(got.cpu().numpy(), ref)
            print(f"  {name} rel L2 {e:.3g}", flush=True)
            assert e <= TOL
        else:
            # the fp32 bound of 1e-5 is for values of order one; at this scale the gradients reach
            # about 12 and fp32 rounding grows with them, so the bound scales with the largest value
            e, m = max_abs(got.cpu().numpy(), ref), float(np.max(np.abs(ref)))
            print(f"  {name} max abs {e:.3g} (largest |value| {m:.3g})", flush=True)
            assert e <= 1e-5 * max(1.0, m)
    for x, y in zip(grads[0], grads[1]):
        assert torch.equal(x, y)
