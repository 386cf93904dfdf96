"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an oracle namespace ``o`` (the real ``oracle`` package,
or a mutant with a planted mistake) and raises AssertionError when the oracle
disagrees with:

* closed forms (Q = 0 gives LSE = ln #allowed and O = mean of the allowed V;
  one key gives O = v_0; constant V is returned unchanged),
* invariants (softmax rows sum to one; token permutations with their
  positions change nothing; gradient identities),
* library routines on special cases (PyTorch's SDPA math path and autograd
  in float64 on the CPU, SciPy's logsumexp),
* a 50-digit Decimal brute force on tiny inputs,
* central finite differences of the forward,
* the memory arithmetic the Accelerate guide prints ("Context Parallel no 🤗
  accelerate", section "Por que paralelismo de contexto?").
"""
from __future__ import annotations

import itertools
import math
from decimal import Decimal, getcontext

import numpy as np

MODES = ("none", "causal", "doc_causal")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _case(rng, B=1, hq=4, hkv=2, s=24, d=8, n_docs=3):
    q, k, v = _rand(rng, B, hq, s, d), _rand(rng, B, hkv, s, d), _rand(rng, B, hkv, s, d)
    pos = np.arange(s)
    cuts = np.sort(rng.choice(np.arange(1, s), n_docs - 1, replace=False))
    cu = np.concatenate([[0], cuts, [s]])
    doc = np.searchsorted(cu, pos, side="right") - 1
    return q, k, v, pos, doc


def _docs(mode, doc):
    return (doc, doc) if mode == "doc_causal" else (None, None)


def _mask_ref(mode, s, doc=None):
    """The mask written out with explicit loops, independent of the oracle's own."""
    m = np.zeros((s, s), dtype=bool)
    for i in range(s):
        for j in range(s):
            if mode == "none":
                m[i, j] = True
            elif mode == "causal":
                m[i, j] = j <= i
            else:
                m[i, j] = j <= i and doc[i] == doc[j]
    return m


# ---------------------------------------------------------------- forward
def pin_constant_v(o):
    rng = np.random.default_rng(10)
    for mode in MODES:
        q, k, v, pos, doc = _case(rng)
        v[:] = 0.375
        out, _ = o.attention_forward(q, k, v, pos, pos, mode, *_docs(mode, doc))
        assert np.max(np.abs(out - 0.375)) <= 1e-14, mode


def pin_rows_sum_to_one(o):
    """V = identity rows: O_i equals row i of the attention weights."""
    rng = np.random.default_rng(11)
    s = 12
    for mode in MODES:
        q, k, _, pos, doc = _case(rng, hq=2, hkv=1, s=s, d=s)
        v = np.broadcast_to(np.eye(s), (1, 1, s, s)).copy()
        p, _ = o.attention_forward(q, k, v, pos, pos, mode, *_docs(mode, doc))
        assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-14, mode
        assert p.min() >= 0.0
        # masked weights are exactly zero; the mask is written out independently here
        if mode == "none":
            banned = np.zeros((s, s), bool)
        elif mode == "causal":
            banned = np.triu(np.ones((s, s), bool), 1)
        else:
            banned = np.triu(np.ones((s, s), bool), 1) | (doc[:, None] != doc[None, :])
        assert np.all(p[0][:, banned] == 0.0), mode
        assert np.all(p[0][:, ~banned] > 0.0), mode


def pin_zero_q(o):
    """Q = 0: every allowed score is 0, so LSE = ln(#allowed) and O = mean of allowed V."""
    rng = np.random.default_rng(12)
    for mode in MODES:
        _, k, v, pos, doc = _case(rng, s=20)
        q = np.zeros((1, 4, 20, 8))
        out, lse = o.attention_forward(q, k, v, pos, pos, mode, *_docs(mode, doc))
        for i in range(20):
            if mode == "none":
                keys = np.arange(20)
            elif mode == "causal":
                keys = np.arange(i + 1)
            else:
                keys = np.nonzero(doc == doc[i])[0]
                keys = keys[keys <= i]
            for h in range(4):
                assert abs(lse[0, h, i] - math.log(keys.size)) <= 1e-13
                ref = v[0, h // 2, keys].mean(axis=0)
                assert np.max(np.abs(out[0, h, i] - ref)) <= 1e-13


def pin_single_key(o):
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 1, 2, 1, 5), _rand(rng, 1, 2, 1, 5), _rand(rng, 1, 2, 1, 5)
    out, lse = o.attention_forward(q, k, v, [7], [7], "causal")
    for h in range(2):
        assert np.max(np.abs(out[0, h, 0] - v[0, h, 0])) <= 1e-15
        assert abs(lse[0, h, 0] - float(q[0, h, 0] @ k[0, h, 0]) / math.sqrt(5)) <= 1e-15


def pin_fully_masked_row(o):
    rng = np.random.default_rng(14)
    q, k, v = _rand(rng, 1, 1, 2, 4), _rand(rng, 1, 1, 3, 4), _rand(rng, 1, 1, 3, 4)
    out, lse = o.attention_forward(q, k, v, [0, 10], [5, 6, 7], "causal")
    assert lse[0, 0, 0] == -np.inf and np.all(out[0, 0, 0] == 0.0)
    assert np.isfinite(lse[0, 0, 1])


def _torch_reference(q, k, v, mask, scale):
    import torch
    import torch.nn.functional as F
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    g = q.shape[1] // k.shape[1]
    kr = tk.repeat_interleave(g, dim=1)
    vr = tv.repeat_interleave(g, dim=1)
    out = F.scaled_dot_product_attention(tq, kr, vr, attn_mask=torch.tensor(mask), scale=scale)
    return torch, tq, tk, tv, out


def pin_torch_sdpa_forward(o):
    """PyTorch's SDPA (CPU, float64) on whole sequences, where every row sees its diagonal."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(15)
    for mode in MODES:
        for d, scale in ((8, None), (16, 0.3)):
            q, k, v, pos, doc = _case(rng, B=2, hq=6, hkv=2, s=33, d=d)
            mask = _mask_ref(mode, 33, doc)
            sc = 1.0 / math.sqrt(d) if scale is None else scale
            _, _, _, _, ref = _torch_reference(q, k, v, mask, sc)
            out, lse = o.attention_forward(q, k, v, pos, pos, mode, *_docs(mode, doc), scale=scale)
            assert np.max(np.abs(out - ref.detach().numpy())) <= 1e-13, (mode, d)
            kr = np.repeat(k, 3, axis=1)
            s = sc * np.einsum("bhid,bhjd->bhij", q, kr)
            ref_lse = logsumexp(np.where(mask, s, -np.inf), axis=-1)
            assert np.max(np.abs(lse - ref_lse)) <= 1e-13, (mode, d)


def pin_permutation_invariance(o):
    rng = np.random.default_rng(16)
    for mode in MODES:
        q, k, v, pos, doc = _case(rng, s=30)
        out, lse = o.attention_forward(q, k, v, pos, pos, mode, *_docs(mode, doc))
        perm = rng.permutation(30)
        dp = None if mode != "doc_causal" else doc[perm]
        out_p, lse_p = o.attention_forward(q[:, :, perm], k[:, :, perm], v[:, :, perm], pos[perm], pos[perm],
                                           mode, dp, dp)
        assert np.max(np.abs(out_p - out[:, :, perm])) <= 1e-13
        assert np.max(np.abs(lse_p - lse[:, :, perm])) <= 1e-13


def pin_skip_masked_columns(o):
    rng = np.random.default_rng(17)
    for mode in MODES:
        q, k, v, pos, doc = _case(rng, s=64, n_docs=5)
        a = o.attention_forward(q, k, v, pos, pos, mode, *_docs(mode, doc), row_block=16)
        b = o.attention_forward(q, k, v, pos, pos, mode, *_docs(mode, doc), row_block=16,
                                skip_masked_columns=True)
        assert np.max(np.abs(a[0] - b[0])) <= 1e-13 and np.max(np.abs(a[1] - b[1])) <= 1e-13
        do = _rand(rng, *q.shape)
        ga = o.attention_backward(q, k, v, do, pos, pos, mode, *_docs(mode, doc), row_block=16)
        gb = o.attention_backward(q, k, v, do, pos, pos, mode, *_docs(mode, doc), row_block=16,
                                  skip_masked_columns=True)
        for x, y in zip(ga, gb):
            assert np.max(np.abs(x - y)) <= 1e-13


# ------------------------------------------------------- Decimal brute force
def _dec_attention(q, k, v, allowed, scale):
    """Row softmax written as exp(s_j) / sum exp(s_k) in 50-digit decimals (no max shift)."""
    getcontext().prec = 50
    sq, sk = len(q), len(k)
    out, lse = [], []
    for i in range(sq):
        ex = []
        for j in range(sk):
            if allowed[i][j]:
                s = scale * sum(Decimal(float(a)) * Decimal(float(b)) for a, b in zip(q[i], k[j]))
                ex.append((j, s.exp()))
        tot = sum(e for _, e in ex)
        lse.append(tot.ln())
        out.append([sum(e * Decimal(float(v[j][c])) for j, e in ex) / tot for c in range(len(v[0]))])
    return out, lse


def pin_decimal_forward(o):
    rng = np.random.default_rng(18)
    for s, d in ((1, 1), (3, 2), (4, 3)):
        q, k, v = _rand(rng, 1, 1, s, d), _rand(rng, 1, 1, s, d), _rand(rng, 1, 1, s, d)
        pos = np.arange(s)
        doc = np.array([0, 0, 1, 1][:s])
        for mode in MODES:
            allowed = _mask_ref(mode, s, doc)
            scale = Decimal(1) / Decimal(d).sqrt()
            ref_o, ref_l = _dec_attention(q[0, 0], k[0, 0], v[0, 0], allowed, scale)
            out, lse = o.attention_forward(q, k, v, pos, pos, mode, *_docs(mode, doc))
            for i in range(s):
                assert abs(Decimal(float(lse[0, 0, i])) - ref_l[i]) <= Decimal("1e-15") * (1 + abs(ref_l[i]))
                for c in range(d):
                    assert abs(Decimal(float(out[0, 0, i, c])) - ref_o[i][c]) <= \
                        Decimal("1e-15") * (1 + abs(ref_o[i][c]))


def _dec_loss(q, k, v, do, allowed, scale):
    out, _ = _dec_attention(q, k, v, allowed, scale)
    return sum(out[i][c] * Decimal(float(do[i][c])) for i in range(len(q)) for c in range(len(do[0])))


def pin_decimal_backward(o):
    """Gradients against 50-digit central differences of the 50-digit loss (step 1e-20)."""
    getcontext().prec = 50
    rng = np.random.default_rng(19)
    s, d = 3, 2
    q, k, v, do = (_rand(rng, 1, 1, s, d) for _ in range(4))
    pos = np.arange(s)
    for mode in ("none", "causal"):
        allowed = _mask_ref(mode, s)
        scale = Decimal(1) / Decimal(d).sqrt()
        grads = o.attention_backward(q, k, v, do, pos, pos, mode)
        h = Decimal("1e-20")
        for which, g in zip((0, 1, 2), grads):
            for i, c in itertools.product(range(s), range(d)):
                mats = [[[Decimal(float(x)) for x in row] for row in m[0, 0]] for m in (q, k, v)]
                mats[which][i][c] += h
                lp = _dec_loss_exact(mats, do[0, 0], allowed, scale)
                mats[which][i][c] -= 2 * h
                lm = _dec_loss_exact(mats, do[0, 0], allowed, scale)
                ref = (lp - lm) / (2 * h)
                assert abs(Decimal(float(g[0, 0, i, c])) - ref) <= Decimal("1e-14") * (1 + abs(ref)), \
                    (mode, which, i, c)


def _dec_loss_exact(mats, do, allowed, scale):
    q, k, v = mats
    tot = Decimal(0)
    for i in range(len(q)):
        ex = []
        for j in range(len(k)):
            if allowed[i][j]:
                ex.append((j, (scale * sum(a * b for a, b in zip(q[i], k[j]))).exp()))
        z = sum(e for _, e in ex)
        for c in range(len(v[0])):
            tot += sum(e * v[j][c] for j, e in ex) / z * Decimal(float(do[i][c]))
    return tot


# ---------------------------------------------------------------- backward
def pin_torch_autograd_backward(o):
    rng = np.random.default_rng(20)
    for mode in MODES:
        q, k, v, pos, doc = _case(rng, B=2, hq=4, hkv=2, s=29, d=8)
        do = _rand(rng, *q.shape)
        mask = _mask_ref(mode, 29, doc)
        torch, tq, tk, tv, out = _torch_reference(q, k, v, mask, 1.0 / math.sqrt(8))
        (out * torch.tensor(do)).sum().backward()
        dq, dk, dv = o.attention_backward(q, k, v, do, pos, pos, mode, *_docs(mode, doc))
        for mine, ref in ((dq, tq), (dk, tk), (dv, tv)):
            assert np.max(np.abs(mine - ref.grad.numpy())) <= 1e-12, mode


def pin_finite_differences(o):
    rng = np.random.default_rng(21)
    q, k, v, pos, doc = _case(rng, hq=2, hkv=1, s=6, d=3, n_docs=2)
    do = _rand(rng, *q.shape)
    for mode in MODES:
        dq, dk, dv = o.attention_backward(q, k, v, do, pos, pos, mode, *_docs(mode, doc))

        def loss(qq, kk, vv):
            out, _ = o.attention_forward(qq, kk, vv, pos, pos, mode, *_docs(mode, doc))
            return float(np.sum(out * do))

        h = 1e-6
        for which, grad in ((0, dq), (1, dk), (2, dv)):
            args = [q, k, v]
            num = np.zeros_like(args[which])
            for idx in np.ndindex(args[which].shape):
                plus = [a.copy() for a in args]
                minus = [a.copy() for a in args]
                plus[which][idx] += h
                minus[which][idx] -= h
                num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
            err = np.linalg.norm(num - grad) / max(np.linalg.norm(grad), 1e-300)
            assert err <= 1e-7, (mode, which, err)


def pin_backward_identities(o):
    rng = np.random.default_rng(22)
    for mode in MODES:
        q, k, v, pos, doc = _case(rng, B=1, hq=4, hkv=2, s=40, d=8)
        do = _rand(rng, *q.shape)
        dq, dk, dv = o.attention_backward(q, k, v, do, pos, pos, mode, *_docs(mode, doc))
        # sum over keys of dS is zero per row -> sum_j dK_j = 0 for every kv head
        assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12, mode
        # sum over keys of P is one per row -> sum_j dV_j = sum over the group's rows of dO
        ref = do.reshape(1, 2, 2, 40, 8).sum(axis=(2, 3))
        assert np.max(np.abs(dv.sum(axis=2) - ref)) <= 1e-12, mode
        # all keys equal -> scores constant along each row -> dQ = 0
        k_eq = np.broadcast_to(k[:, :, :1], k.shape).copy()
        dq0, _, _ = o.attention_backward(q, k_eq, v, do, pos, pos, mode, *_docs(mode, doc))
        assert np.max(np.abs(dq0)) <= 1e-12, mode


def pin_gqa_equals_repeated_mha(o):
    rng = np.random.default_rng(23)
    for mode in MODES:
        q, k, v, pos, doc = _case(rng, hq=6, hkv=2, s=20)
        do = _rand(rng, *q.shape)
        out, lse = o.attention_forward(q, k, v, pos, pos, mode, *_docs(mode, doc))
        kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
        out_r, lse_r = o.attention_forward(q, kr, vr, pos, pos, mode, *_docs(mode, doc))
        assert np.max(np.abs(out - out_r)) <= 1e-13 and np.max(np.abs(lse - lse_r)) <= 1e-13
        dq, dk, dv = o.attention_backward(q, k, v, do, pos, pos, mode, *_docs(mode, doc))
        dq_r, dk_r, dv_r = o.attention_backward(q, kr, vr, do, pos, pos, mode, *_docs(mode, doc))
        assert np.max(np.abs(dq - dq_r)) <= 1e-13
        assert np.max(np.abs(dk - dk_r.reshape(1, 2, 3, 20, 8).sum(2))) <= 1e-13
        assert np.max(np.abs(dv - dv_r.reshape(1, 2, 3, 20, 8).sum(2))) <= 1e-13


# ---------------------------------------------------------------- ring / merge
def pin_ring_equals_plain(o):
    """Ring-merged blockwise attention equals unsharded attention to 1e-12."""
    rng = np.random.default_rng(24)
    for n in (1, 2, 4, 8):
        for scheme in ("contiguous", "zigzag"):
            for mode in MODES:
                s = 2 * n * 5
                q, k, v, pos, doc = _case(rng, hq=4, hkv=2, s=s, d=8, n_docs=4 if s > 4 else 1)
                dd = doc if mode == "doc_causal" else None
                ref_o, ref_l = o.attention_forward(q, k, v, pos, pos, mode, dd, dd)
                out, lse = o.ring_forward(q, k, v, pos, mode, n, scheme, doc=dd)
                assert np.max(np.abs(out - ref_o)) <= 1e-12, (n, scheme, mode)
                assert np.max(np.abs(lse - ref_l)) <= 1e-12, (n, scheme, mode)


def pin_ring_step_order(o):
    rng = np.random.default_rng(25)
    q, k, v, pos, doc = _case(rng, hq=2, hkv=1, s=48, d=8, n_docs=5)
    a = o.ring_forward(q, k, v, pos, "doc_causal", 4, "zigzag", doc=doc)
    b = o.ring_forward(q, k, v, pos, "doc_causal", 4, "zigzag", doc=doc,
                       step_order=lambda r, n: [(r + t) % n for t in range(n)][::-1])
    assert np.max(np.abs(a[0] - b[0])) <= 1e-13 and np.max(np.abs(a[1] - b[1])) <= 1e-13


def pin_merge_identity_and_closed_form(o):
    rng = np.random.default_rng(26)
    oa = rng.standard_normal((3, 4))
    la = rng.standard_normal(3)
    ob = rng.standard_normal((3, 4))
    lb = rng.standard_normal(3)
    empty_o, empty_l = np.zeros((3, 4)), np.full(3, -np.inf)
    m, l = o.merge(oa, la, empty_o, empty_l)
    assert np.array_equal(m, oa) and np.array_equal(l, la)
    m, l = o.merge(empty_o, empty_l, ob, lb)
    assert np.array_equal(m, ob) and np.array_equal(l, lb)
    m, l = o.merge(empty_o, empty_l, empty_o, empty_l)
    assert np.all(m == 0) and np.all(l == -np.inf)
    # two halves of one softmax: weights are the halves' shares of the total mass
    m, l = o.merge(oa, la, ob, lb)
    wa = np.exp(la) / (np.exp(la) + np.exp(lb))
    assert np.max(np.abs(l - np.log(np.exp(la) + np.exp(lb)))) <= 1e-14
    assert np.max(np.abs(m - (wa[:, None] * oa + (1 - wa)[:, None] * ob))) <= 1e-14


def pin_shards(o):
    for n in (1, 2, 4, 8):
        s = 16 * n
        for scheme in ("contiguous", "zigzag"):
            sh = o.shard_rows(s, n, scheme)
            assert all(x.size == s // n for x in sh)
            assert np.array_equal(np.sort(np.concatenate(sh)), np.arange(s))
        c = s // (2 * n)
        zz = o.shard_rows(s, n, "zigzag")
        for r in range(n):
            assert np.array_equal(zz[r][:c], np.arange(r * c, (r + 1) * c))
            assert np.array_equal(zz[r][c:], np.arange((2 * n - 1 - r) * c, (2 * n - r) * c))


def zigzag_pairs_closed_form(n, c, r, j):
    """Allowed causal pairs of rank r's zigzag Q shard against block j (chunks of c tokens)."""
    return 2 * c * c + (c if j == r else 0)


def pin_zigzag_balance(o):
    for n, c in ((2, 3), (4, 5), (8, 2)):
        s = 2 * n * c
        sh = o.shard_rows(s, n, "zigzag")
        for r in range(n):
            tot = 0
            for j in range(n):
                p = o.count_allowed_pairs(sh[r], sh[j], "causal")
                assert p == zigzag_pairs_closed_form(n, c, r, j), (n, c, r, j)
                tot += p
            assert tot == 2 * n * c * c + c
        assert sum(o.count_allowed_pairs(sh[r], np.arange(s), "causal") for r in range(n)) == s * (s + 1) // 2


def pin_docs_from_cu_seqlens(o):
    cu = np.array([0, 3, 4, 10])
    assert list(o.docs_from_cu_seqlens(cu, 10)) == [0, 0, 0, 1, 2, 2, 2, 2, 2, 2]


ALL_PINS = [pin_constant_v, pin_rows_sum_to_one, pin_zero_q, pin_single_key, pin_fully_masked_row,
            pin_torch_sdpa_forward, pin_permutation_invariance, pin_skip_masked_columns,
            pin_decimal_forward, pin_decimal_backward, pin_torch_autograd_backward,
            pin_finite_differences, pin_backward_identities, pin_gqa_equals_repeated_mha,
            pin_ring_equals_plain, pin_ring_step_order, pin_merge_identity_and_closed_form,
            pin_shards, pin_zigzag_balance, pin_docs_from_cu_seqlens]
