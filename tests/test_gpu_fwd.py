"""Forward parity on the GPU: the HIP path through the C ABI against the fp64 oracle.

Tolerances: fp32 problems max |err| <= 1e-5 on O and LSE; bf16 problems
max |err| <= 1e-2 on O (bf16 output and fp32 running output) and <= 1e-3 on
LSE.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import ring_attention_ringattn_amd as ra
import synthetic
from tests.gpu_util import rel_l2, Ring, dev, max_abs, oracle_rows, print_case, thd_view, MASKS, TORCH_DT

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "bf16": (1e-2, 1e-3)}


def _check_rank(ring, i, r, O, L, dtype, rows_idx=None):
    tol_o, tol_l = TOL[dtype]
    sel = slice(None) if rows_idx is None else rows_idx
    out = ring.numpy("out")[i][:, :, sel]
    o_acc = ring.numpy("o_acc")[i][:, :, sel]
    lse = ring.numpy("lse")[i][:, :, sel]
    assert np.all(np.isfinite(out)), "output not fully written"
    e_out, e_acc, e_lse = max_abs(out, O), max_abs(o_acc, O), max_abs(lse, L)
    print(f"  rank {r}: max|dO| out {e_out:.3g} o_acc {e_acc:.3g} max|dLSE| {e_lse:.3g}", flush=True)
    assert e_out <= tol_o and e_acc <= tol_o and e_lse <= tol_l


def test_c1_fp32_contiguous_causal_all_ranks():
    w = synthetic.WORKLOADS["c1"]
    print_case("c1: fp32, 2 heads, D=64, S=512, 4 contiguous shards, causal")
    inp = synthetic.make_inputs(w)
    pos = ra.sharding.shard_positions(w.seq, w.n_shards, w.sharding)
    ring = Ring(inp["q"], inp["k"], inp["v"], pos, "causal", "f32", w.ranks()).forward()
    O, L = oracle.attention_forward(inp["q"], inp["k"], inp["v"], np.arange(w.seq), np.arange(w.seq), "causal")
    for i, r in enumerate(ring.ranks):
        _check_rank(ring, i, r, O[:, :, pos[r]], L[:, :, pos[r]], "f32")


def test_c2_bf16_zigzag_gqa_all_ranks():
    w = synthetic.WORKLOADS["c2"]
    print_case("c2: bf16, 32/8 GQA, D=128, S=8192, 4 zigzag shards, causal")
    inp = synthetic.make_inputs(w)
    pos = ra.sharding.shard_positions(w.seq, w.n_shards, w.sharding)
    ring = Ring(inp["q"], inp["k"], inp["v"], pos, "causal", "bf16", w.ranks()).forward()
    O, L = oracle.attention_forward(inp["q"], inp["k"], inp["v"], np.arange(w.seq), np.arange(w.seq), "causal",
                                    row_block=256, skip_masked_columns=True)
    for i, r in enumerate(ring.ranks):
        _check_rank(ring, i, r, O[:, :, pos[r]], L[:, :, pos[r]], "bf16")



def test_long_ring_many_tile_tables():
    """A 50-rank ring (more tile tables than one batched table launch takes): ranks 47-49 emulated,
    zigzag, 6400 tokens, 4/2 heads, D = 64, forward and backward against the oracle."""
    w = synthetic.small_workload("c2", seq=6400, n_shards=50, hq=4, hkv=2, head_dim=64, seed=50,
                                 emulated_ranks=(47, 48, 49), backward=True)
    print_case("long ring: 50 zigzag ranks of 128 tokens, ranks 47-49, 4/2 heads, D=64, fwd + bwd")
    inp = synthetic.make_inputs(w)
    pos = ra.sharding.shard_positions(w.seq, w.n_shards, w.sharding)
    ring = Ring(inp["q"], inp["k"], inp["v"], pos, "causal", "bf16", w.ranks(), do_glob=inp["do"])
    ring.forward().backward()
    s_all = np.arange(w.seq)
    O, L = oracle.attention_forward(inp["q"], inp["k"], inp["v"], s_all, s_all, "causal", skip_masked_columns=True)
    for i, r in enumerate(ring.ranks):
        _check_rank(ring, i, r, O[:, :, pos[r]], L[:, :, pos[r]], "bf16")
    rows = np.concatenate([pos[r] for r in ring.ranks])
    dQ, dK, dV = oracle.attention_backward(inp["q"][:, :, rows], inp["k"], inp["v"], inp["do"][:, :, rows], rows,
                                           s_all, "causal", skip_masked_columns=True)
    off = 0
    for i, r in enumerate(ring.ranks):
        n = pos[r].size
        assert rel_l2(ring.numpy("dq")[i], dQ[:, :, off:off + n]) <= 2e-2
        off += n
    dk = np.concatenate(ring.numpy("dk"), axis=2)
    dv = np.concatenate(ring.numpy("dv"), axis=2)
    order = np.concatenate(pos)
    assert rel_l2(dk, dK[:, :, order]) <= 2e-2 and rel_l2(dv, dV[:, :, order]) <= 2e-2

def _sampled_rows(pos_rank, c, rng, n=48):
    """Random rows plus the first/last row of each chunk and of each 64-row tile edge nearby."""
    idx = set(rng.choice(pos_rank.size, n, replace=False).tolist())
    for k in range(0, pos_rank.size, c):
        idx.update([k, k + 1, k + 63, k + 64, k + c - 1])
    return np.array(sorted(i for i in idx if 0 <= i < pos_rank.size))


@pytest.mark.parametrize("rank", [0, 4, 7])
def test_c3_full_size_one_rank_sampled_rows(rank):
    """One rank's share of a 131072-token context over 8 zigzag blocks, prefetch on; exact per sampled row.

    Ranks 0, N/2 and N-1: each holds a different mix of full, partial and empty tiles per step."""
    w = synthetic.WORKLOADS["c3"]
    print_case(f"c3: bf16 rank {rank} of 8, 16384 local queries, 8 steps of 16384 keys, zigzag causal")
    pos = ra.sharding.shard_positions(w.seq, w.n_shards, w.sharding)
    inp = synthetic.make_inputs(w, q_rows=pos[rank])
    ring = Ring(None, inp["k"], inp["v"], pos, "causal", "bf16", [rank], q_shards=[inp["q"]]).forward()
    rows_local = _sampled_rows(pos[rank], w.seq // (2 * w.n_shards), np.random.default_rng(100 + rank))
    O, L = oracle_rows(inp, pos[rank][rows_local], "causal")
    _check_rank(ring, 0, rank, O, L, "bf16", rows_local)


CASES = [
    # dtype, D, B, hq, hkv, sq, sk, mask
    ("bf16", 128, 1, 4, 1, 200, 333, "causal"),
    ("bf16", 128, 2, 2, 2, 130, 64, "none"),
    ("bf16", 64, 1, 6, 3, 257, 190, "doc_causal"),
    ("bf16", 64, 2, 2, 1, 64, 1000, "none"),
    ("f32", 128, 1, 2, 1, 100, 150, "causal"),
    ("f32", 64, 2, 3, 3, 65, 70, "doc_causal"),
    # long enough key blocks (>= 5 tiles) that tiles stream in while others are being used
    ("bf16", 128, 1, 4, 2, 300, 1100, "causal"),
    ("bf16", 128, 1, 4, 2, 300, 1100, "doc_causal"),
    ("bf16", 64, 1, 4, 2, 300, 1100, "doc_causal"),
    # token-major [S, H, D] storage (strided views)
    ("bf16", 128, 1, 4, 2, 300, 1100, "causal", "thd"),
    ("bf16", 128, 1, 4, 2, 300, 1100, "doc_causal", "thd"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_step_fwd_ragged_edges(case):
    """Two manual steps (FIRST, then LAST) over ragged sizes with scattered positions and documents."""
    dtype, d, B, hq, hkv, sq, sk, mask = case[:8]
    layout = case[8] if len(case) > 8 else "bhsd"
    print_case(f"step_fwd {case}")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    wdt = torch.float32 if dtype == "f32" else torch.bfloat16
    # values as in the workloads: bf16 inputs N(0,1)*0.5, fp32 inputs N(0,1)
    rnd = lambda *s: synthetic.bf16_round(0.5 * rng.standard_normal(s).astype(np.float32)) if dtype == "bf16" \
        else rng.standard_normal(s).astype(np.float32)
    q = rnd(B, hq, sq, d)
    k1, v1, k2, v2 = rnd(B, hkv, sk, d), rnd(B, hkv, sk, d), rnd(B, hkv, sk, d), rnd(B, hkv, sk, d)
    tot = sq + 2 * sk
    perm = rng.permutation(tot).astype(np.int32)
    qp, kp1, kp2 = perm[:sq], perm[sq:sq + sk], perm[sq + sk:]
    docs = (np.sort(rng.integers(0, 5, tot)).astype(np.int32))   # document id by position
    qd, kd1, kd2 = docs[qp], docs[kp1], docs[kp2]
    o_acc = torch.zeros(B, hq, sq, d, device="cuda")
    lse = torch.zeros(B, hq, sq, device="cuda")
    out = torch.full((B, hq, sq, d), float("nan"), dtype=wdt, device="cuda")
    dm = mask == "doc_causal"
    put = (lambda a: thd_view(dev(a, wdt))) if layout == "thd" else (lambda a: dev(a, wdt))
    if layout == "thd":
        out = thd_view(out)
    for step, (k, v, kp, kd) in enumerate(((k1, v1, kp1, kd1), (k2, v2, kp2, kd2))):
        ra.ringattn_step_fwd(put(q), put(k), put(v), o_acc, lse, out, dev(qp, torch.int32),
                             dev(kp, torch.int32), dev(qd, torch.int32) if dm else None,
                             dev(kd, torch.int32) if dm else None, mask_mode=MASKS[mask],
                             flags=ra.RA_STEP_FIRST if step == 0 else ra.RA_STEP_LAST)
    torch.cuda.synchronize()
    O, L = oracle.attention_forward(q, np.concatenate([k1, k2], 2), np.concatenate([v1, v2], 2), qp,
                                    np.concatenate([kp1, kp2]), mask, qd if dm else None,
                                    np.concatenate([kd1, kd2]) if dm else None)
    fin = np.isfinite(L)
    got_l = lse.cpu().numpy()
    assert np.array_equal(np.isfinite(got_l), fin), "fully masked rows must have lse = -inf"
    tol_o, tol_l = TOL[dtype]
    assert max_abs(got_l[fin], L[fin]) <= tol_l
    assert max_abs(o_acc.cpu().numpy(), O) <= tol_o          # masked rows: O = 0 on both sides
    assert max_abs(out.float().cpu().numpy(), O) <= tol_o


def test_step_fwd_wide_token_stride():
    """Keys 8 MiB apart (a token stride of 4 Mi elements): the K rows of the 5-tile block span more
    than 2^31 bytes, past what one 31-bit buffer offset reaches, so each key tile is loaded
    through a buffer resource of its own."""
    print_case("step_fwd bf16, D=128, sk=300 keys with a token stride of 4 Mi elements")
    rng = np.random.default_rng(77)
    rnd = lambda *s: synthetic.bf16_round(0.5 * rng.standard_normal(s).astype(np.float32))
    hq, sq, sk, d, stride = 2, 130, 300, 128, 4 << 20
    assert 5 * 64 * stride * 2 >= 2 ** 31
    q, k, v = rnd(1, hq, sq, d), rnd(1, 1, sk, d), rnd(1, 1, sk, d)
    perm = rng.permutation(sq + sk).astype(np.int32)
    qp, kp = perm[:sq], perm[sq:]

    def wide(a):
        n = (sk - 1) * stride + d
        buf = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
        view = buf.as_strided((1, 1, sk, d), (n, n, stride, 1))
        view.copy_(dev(a, torch.bfloat16))
        return view
    kw, vw = wide(k), wide(v)
    o_acc = torch.zeros(1, hq, sq, d, device="cuda")
    lse = torch.zeros(1, hq, sq, device="cuda")
    out = torch.full((1, hq, sq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    ra.ringattn_step_fwd(dev(q, torch.bfloat16), kw, vw, o_acc, lse, out, dev(qp, torch.int32), dev(kp, torch.int32),
                         mask_mode=ra.RA_MASK_CAUSAL, flags=ra.RA_STEP_FIRST | ra.RA_STEP_LAST)
    torch.cuda.synchronize()
    O, L = oracle.attention_forward(q, k, v, qp, kp, "causal")
    fin = np.isfinite(L)
    got_l = lse.cpu().numpy()
    assert np.array_equal(np.isfinite(got_l), fin)
    assert max_abs(got_l[fin], L[fin]) <= 1e-3
    assert max_abs(o_acc.cpu().numpy(), O) <= 1e-2
    assert max_abs(out.float().cpu().numpy(), O) <= 1e-2
    del kw, vw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d", [128, 64])
def test_step_fwd_tile_lists_with_gaps(d):
    """Document-causal step of the last of 4 contiguous shards against its own block: the
    non-empty key tiles of a query tile start past tile 0 and skip tiles (documents end)."""
    print_case(f"step_fwd doc-causal diagonal block, D={d}")
    rng = np.random.default_rng(5)
    rnd = lambda *s: synthetic.bf16_round(0.5 * rng.standard_normal(s).astype(np.float32))
    cu = np.array([0, 313, 1847, 3151, 3314, 3524, 3683, 4096], np.int32)
    doc = oracle.docs_from_cu_seqlens(cu, 4096)
    p = np.arange(3072, 4096, dtype=np.int32)
    q, k, v = rnd(1, 4, 1024, d), rnd(1, 2, 1024, d), rnd(1, 2, 1024, d)
    o = torch.zeros(1, 4, 1024, d, device="cuda")
    lse = torch.zeros(1, 4, 1024, device="cuda")
    bf = torch.bfloat16
    ra.ringattn_step_fwd(dev(q, bf), dev(k, bf), dev(v, bf), o, lse, None, dev(p, torch.int32), dev(p, torch.int32),
                         dev(doc[p], torch.int32), dev(doc[p], torch.int32), mask_mode=ra.RA_MASK_DOC_CAUSAL,
                         flags=ra.RA_STEP_FIRST)
    torch.cuda.synchronize()
    O, L = oracle.attention_forward(q, k, v, p, p, "doc_causal", doc[p], doc[p])
    assert max_abs(lse.cpu().numpy(), L) <= 1e-3
    assert max_abs(o.cpu().numpy(), O) <= 1e-2


def test_empty_and_fully_masked():
    print_case("empty query shard, empty key block, block entirely after the queries")
    q = torch.zeros(1, 2, 0, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16, device="cuda")
    ra.ringattn_step_fwd(q, k, k, torch.zeros(1, 2, 0, 128, device="cuda"), torch.zeros(1, 2, 0, device="cuda"),
                         None, torch.zeros(0, dtype=torch.int32, device="cuda"),
                         torch.zeros(64, dtype=torch.int32, device="cuda"), flags=ra.RA_STEP_FIRST)
    # sk = 0 with FIRST|LAST: identity partial -> o = 0, lse = -inf
    q = torch.ones(1, 2, 70, 128, dtype=torch.bfloat16, device="cuda")
    k0 = torch.zeros(1, 2, 0, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.full((1, 2, 70, 128), 5.0, device="cuda")
    l = torch.full((1, 2, 70), 5.0, device="cuda")
    out = torch.full((1, 2, 70, 128), 5.0, dtype=torch.bfloat16, device="cuda")
    qp = torch.arange(70, dtype=torch.int32, device="cuda")
    ra.ringattn_step_fwd(q, k0, k0, o, l, out, qp, torch.zeros(0, dtype=torch.int32, device="cuda"),
                         flags=ra.RA_STEP_FIRST | ra.RA_STEP_LAST)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(l == float("-inf")) and torch.all(out == 0)
    # a block entirely in the future of every query: the running result is unchanged
    o_prev = torch.randn(1, 2, 70, 128, device="cuda")
    l_prev = torch.randn(1, 2, 70, device="cuda")
    o2, l2 = o_prev.clone(), l_prev.clone()
    kf = torch.randn(1, 2, 64, 128, device="cuda").to(torch.bfloat16)
    ra.ringattn_step_fwd(q, kf, kf, o2, l2, None, qp, torch.arange(1000, 1064, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o2, o_prev) and torch.equal(l2, l_prev)


def _small_zigzag_ring(n=4, seq=2048, seed=7, mask="causal", ranks=None):
    w = synthetic.small_workload("c2", seq=seq, n_shards=n, hq=8, hkv=2, seed=seed)
    inp = synthetic.make_inputs(w)
    pos = ra.sharding.shard_positions(w.seq, n, "zigzag")
    return Ring(inp["q"], inp["k"], inp["v"], pos, mask, "bf16", ranks if ranks is not None else range(n)), inp, pos


def test_run_modes_are_bitwise_equal():
    """Overlapped prefetch, serial copies, DMA-engine copies, poisoned slots and no tile skipping
    give identical bits."""
    print_case("run modes: overlapped vs serial vs DMA engine vs poison vs no-skip, 8-rank zigzag, all ranks")
    ring, _, _ = _small_zigzag_ring(n=8, seq=4096)
    ring.forward()
    ref = [t.clone() for t in ring.o_acc], [t.clone() for t in ring.lse], [t.clone() for t in ring.out]
    for flags, cs in ((ra.RA_RUN_SERIAL_COPY, "side"), (0, None), (ra.RA_RUN_POISON, "side"),
                      (ra.RA_RUN_COPY_ENGINE, "side"), (ra.RA_RUN_COPY_ENGINE | ra.RA_RUN_POISON, "side"),
                      (ra.RA_NO_SKIP, "side")):
        print(f"  flags {flags} copy stream {cs}", flush=True)
        ring.forward(flags=flags, copy_stream=cs)
        for a, b in zip(ring.o_acc, ref[0]):
            assert torch.equal(a, b)
        for a, b in zip(ring.lse, ref[1]):
            assert torch.equal(a, b)
        for a, b in zip(ring.out, ref[2]):
            assert torch.equal(a, b)


def test_merge_kernel_mode_matches_fused_merge():
    print_case("run with the standalone merge kernel vs the merge fused in the step kernel")
    ring, inp, pos = _small_zigzag_ring(n=4, seq=2048)
    ring.forward()
    ref_o, ref_l = [t.clone() for t in ring.o_acc], [t.clone() for t in ring.lse]
    ring.forward(flags=ra.RA_RUN_MERGE_KERNEL)
    for a, b in zip(ring.o_acc, ref_o):
        assert torch.max(torch.abs(a - b)).item() <= 2e-6
    for a, b in zip(ring.lse, ref_l):
        assert torch.max(torch.abs(a - b)).item() <= 2e-6
    O, L = oracle.attention_forward(inp["q"], inp["k"], inp["v"], np.arange(2048), np.arange(2048), "causal")
    for i, r in enumerate(ring.ranks):
        assert max_abs(ring.numpy("out")[i], O[:, :, pos[r]]) <= 1e-2


def test_resume_from_checkpoint_is_bitwise_equal():
    """(o_acc, lse) after step t is a checkpoint: clobber the staging state, resume, get the same bits."""
    print_case("resume after step 3 of 8")
    ring, _, _ = _small_zigzag_ring(n=8, seq=4096)
    ring.forward()
    ref_o, ref_l, ref_out = [t.clone() for t in ring.o_acc], [t.clone() for t in ring.lse], \
        [t.clone() for t in ring.out]
    ring.forward(stop_step=3)
    saved = [t.cpu() for t in ring.o_acc], [t.cpu() for t in ring.lse]
    for t in ring.o_acc + ring.lse:
        t.fill_(float("nan"))
    for t, s in zip(ring.o_acc, saved[0]):
        t.copy_(s)
    for t, s in zip(ring.lse, saved[1]):
        t.copy_(s)
    ring.forward(start_step=3, alloc=False)
    for a, b in zip(ring.o_acc + ring.lse + ring.out, ref_o + ref_l + ref_out):
        assert torch.equal(a, b)


def test_merge_entry_point():
    print_case("ringattn_merge against the oracle's merge, with -inf rows")
    rng = np.random.default_rng(3)
    for d in (64, 128):
        oa, ob = rng.standard_normal((2, 3, 77, d)), rng.standard_normal((2, 3, 77, d))
        la, lb = rng.standard_normal((2, 3, 77)) * 4, rng.standard_normal((2, 3, 77)) * 4
        la[0, 0, :5] = -np.inf
        lb[0, 1, :5] = -np.inf
        la[1, 2, :3] = lb[1, 2, :3] = -np.inf
        oa[la == -np.inf] = 0
        ob[lb == -np.inf] = 0
        ta, tla = dev(oa), dev(la)
        tb, tlb = dev(ob), dev(lb)
        ra.ringattn_merge(ta, tla, tb, tlb)
        torch.cuda.synchronize()
        ro, rl = oracle.merge(oa.astype(np.float32).astype(np.float64), la.astype(np.float32).astype(np.float64),
                              ob.astype(np.float32).astype(np.float64), lb.astype(np.float32).astype(np.float64))
        got_l = tlb.cpu().numpy()
        assert np.array_equal(np.isfinite(got_l), np.isfinite(rl))
        assert max_abs(got_l[np.isfinite(rl)], rl[np.isfinite(rl)]) <= 1e-5
        assert max_abs(tb.cpu().numpy(), ro) <= 1e-5



def test_merge_full_size_sampled_rows():
    """ringattn_merge at the 131072-token share's shape (16384 rows x 32 heads, D = 128), the launch
    the benchmark times: sampled rows against the oracle's merge, every row finite."""
    print_case("ringattn_merge, 1 x 32 x 16384 x 128 fp32 partials")
    rng = np.random.default_rng(31)
    shp = (1, 32, 16384, 128)
    oa = rng.standard_normal(shp, dtype=np.float32)
    ob = rng.standard_normal(shp, dtype=np.float32)
    la = (rng.standard_normal(shp[:3]) * 4).astype(np.float32)
    lb = (rng.standard_normal(shp[:3]) * 4).astype(np.float32)
    la[0, 3, :100] = -np.inf
    oa[0, 3, :100] = 0
    ta, tla, tb, tlb = dev(oa), dev(la), dev(ob), dev(lb)
    ra.ringattn_merge(ta, tla, tb, tlb)
    torch.cuda.synchronize()
    got_o, got_l = tb.cpu().numpy(), tlb.cpu().numpy()
    assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_l))
    heads = np.arange(32)
    rows = np.unique(np.concatenate([rng.choice(16384, 64, replace=False), [0, 1, 99, 100, 16383]]))
    sel = np.ix_([0], heads, rows)
    f64 = lambda x: x.astype(np.float64)
    ro, rl = oracle.merge(f64(oa[sel]), f64(la[sel]), f64(ob[sel]), f64(lb[sel]))
    assert max_abs(got_l[sel], rl) <= 1e-5
    assert max_abs(got_o[sel], ro) <= 1e-5

def test_thd_layout_doc_causal():
    """Packed [T, H, D] token-major storage (strided views) with a document-causal mask."""
    print_case("THD layout, doc-causal, 4 contiguous shards of a 4096-token packed stream")
    w = synthetic.small_workload("c5", seq=4096, n_shards=4, hq=4, hkv=2)
    inp = synthetic.make_inputs(w, backward=False)
    cu = synthetic.doc_lengths(11, 4096, median=300.0)
    cu = np.concatenate([[0], np.cumsum(cu)]).astype(np.int32)
    doc = oracle.docs_from_cu_seqlens(cu, 4096)
    pos = ra.sharding.shard_positions(4096, 4, "contiguous")
    ring = Ring(inp["q"], inp["k"], inp["v"], pos, "doc_causal", "bf16", range(4), doc=doc, layout="thd")
    # the device doc ids come from the library's own cu_seqlens conversion
    tcu = dev(cu, torch.int32)
    ring.q_doc = [ra.ringattn_docs_from_cu_seqlens(tcu, int(pos[r][0]), pos[r].size) for r in ring.ranks]
    ring.kv_doc = [ra.ringattn_docs_from_cu_seqlens(tcu, int(p[0]), p.size) for p in pos]
    ring.forward()
    O, L = oracle.attention_forward(inp["q"], inp["k"], inp["v"], np.arange(4096), np.arange(4096), "doc_causal",
                                    doc, doc, skip_masked_columns=True)
    for i, r in enumerate(ring.ranks):
        assert np.array_equal(ring.q_doc[i].cpu().numpy(), doc[pos[r]])
        _check_rank(ring, i, r, O[:, :, pos[r]], L[:, :, pos[r]], "bf16")
