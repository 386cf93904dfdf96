"""Plain fp64 attention: the definition the ring method must reproduce.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module;
only the tests, the smoke check and the benchmark's CPU-baseline leg do.

What it computes (global token order, no blocking of the math):

* Scores s_ij = scale * <Q_i, K_j> with scale = 1/sqrt(D) unless given (the
  pages use SDPA, whose default scale this is: the Accelerate guide, "Context
  Parallel no 🤗 accelerate", section "Como usar paralelismo de contexto?", the
  SDPA-only remark).
* Mask (same guide, same remark: no mask or a causal mask; plus the packed
  THD layout with cu_seqlens of the Dynamic-CP page, "Optimización del
  entrenamiento variable con Dynamic Context Parallelism en Megatron Core",
  section "Reprogramación dinámica y empaquetado de datos", read as "same
  document and causal"):
    none        every pair allowed
    causal      pos_k <= pos_q   (inclusive diagonal, global positions)
    doc_causal  causal and doc_k == doc_q
* Softmax over the allowed keys of each row, exactly as vanilla attention
  materialises it (the Accelerate guide, section "Por que paralelismo de
  contexto?": the full score matrix of vanilla attention), LSE_i = ln sum_j
  exp(s_ij), and
  O_i = sum_j P_ij V_j.  A row with no allowed key has LSE = -inf, O = 0.
* GQA: q-head h reads kv-head floor(h * Hkv / Hq).
* Backward of L = sum(O * dO): D_i = <dO_i, O_i>, dP_ij = <dO_i, V_j>,
  dS_ij = P_ij (dP_ij - D_i), dQ_i = scale sum_j dS_ij K_j,
  dK_j = scale sum_{h in group} sum_i dS_ij Q_i,
  dV_j = sum_{h in group} sum_i P_ij dO_i.

Rows are processed in blocks of at most ``row_block`` rows only to bound
memory; each row's softmax is taken over its whole row of scores at once.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

NONE, CAUSAL, DOC_CAUSAL = "none", "causal", "doc_causal"


def allowed_pairs(q_pos, k_pos, mode, q_doc=None, k_doc=None):
    """Boolean [len(q_pos), len(k_pos)] matrix: may query i attend to key j."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    if mode == NONE:
        return np.ones((q_pos.size, k_pos.size), dtype=bool)
    causal = k_pos[None, :] <= q_pos[:, None]
    if mode == CAUSAL:
        return causal
    if mode == DOC_CAUSAL:
        q_doc = np.asarray(q_doc, dtype=np.int64)
        k_doc = np.asarray(k_doc, dtype=np.int64)
        return causal & (k_doc[None, :] == q_doc[:, None])
    raise ValueError(f"unknown mask mode {mode!r}")


def docs_from_cu_seqlens(cu, n_tokens):
    """Document id of every token of a packed stream: doc[t] = k for cu[k] <= t < cu[k+1]."""
    cu = np.asarray(cu, dtype=np.int64)
    doc = np.empty(n_tokens, dtype=np.int64)
    for k in range(cu.size - 1):
        doc[cu[k]:cu[k + 1]] = k
    return doc


def _kv_head(h, hq, hkv):
    return (h * hkv) // hq


def _column_subset(allowed_rows, skip_masked_columns):
    if not skip_masked_columns:
        return slice(None)
    return np.nonzero(allowed_rows.any(axis=0))[0]


def _softmax_rows(s, allowed):
    """Exact row softmax of the allowed entries of s. Returns (P, LSE)."""
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for masked entries
    l = e.sum(axis=1)
    lse = np.where(has, m_safe + np.log(np.where(has, l, 1.0)), -np.inf)
    p = e / np.where(has, l, 1.0)[:, None]
    return p, lse


def attention_forward(q, k, v, q_pos, k_pos, mode, q_doc=None, k_doc=None, scale=None,
                      row_block=64, skip_masked_columns=False):
    """O [B,Hq,Sq,D] and LSE [B,Hq,Sq] in fp64.

    ``q`` [B,Hq,Sq,D] and ``k``/``v`` [B,Hkv,Sk,D] may be any real dtype; they
    are widened to fp64.  ``skip_masked_columns`` drops key columns that no
    row of a block may see; those columns contribute exp(-inf) = 0 terms, so
    the result is the same (a pinned test checks this).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, hq, sq, d = q.shape
    hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((B, hq, sq, d))
    lse = np.full((B, hq, sq), -np.inf)
    for r0 in range(0, sq, row_block):
        rows = slice(r0, min(sq, r0 + row_block))
        allowed = allowed_pairs(np.asarray(q_pos)[rows], k_pos, mode,
                                None if q_doc is None else np.asarray(q_doc)[rows], k_doc)
        cols = _column_subset(allowed, skip_masked_columns)
        allowed = allowed[:, cols]
        for b in range(B):
            for h in range(hq):
                kh = _kv_head(h, hq, hkv)
                s = scale * (q[b, h, rows] @ k[b, kh][cols].T)
                p, lse_blk = _softmax_rows(s, allowed)
                o[b, h, rows] = p @ v[b, kh][cols]
                lse[b, h, rows] = lse_blk
    return o, lse


def attention_backward(q, k, v, do, q_pos, k_pos, mode, q_doc=None, k_doc=None, scale=None,
                       row_block=64, skip_masked_columns=False):
    """(dQ, dK, dV) in fp64 for the loss sum(O * dO), O from attention_forward's definition.

    Query rows whose dO is zero contribute nothing, so a caller that wants one
    shard's contribution passes only that shard's rows (q, do, q_pos, q_doc).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, hq, sq, d = q.shape
    hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, sq, row_block):
        rows = slice(r0, min(sq, r0 + row_block))
        allowed = allowed_pairs(np.asarray(q_pos)[rows], k_pos, mode,
                                None if q_doc is None else np.asarray(q_doc)[rows], k_doc)
        cols = _column_subset(allowed, skip_masked_columns)
        allowed = allowed[:, cols]
        for b in range(B):
            for h in range(hq):
                kh = _kv_head(h, hq, hkv)
                kc, vc = k[b, kh][cols], v[b, kh][cols]
                s = scale * (q[b, h, rows] @ kc.T)
                p, _ = _softmax_rows(s, allowed)
                o_rows = p @ vc
                delta = np.sum(do[b, h, rows] * o_rows, axis=1)
                dp = do[b, h, rows] @ vc.T
                ds = p * (dp - delta[:, None])
                dq[b, h, rows] = scale * (ds @ kc)
                if isinstance(cols, slice):
                    dk[b, kh] += scale * (ds.T @ q[b, h, rows])
                    dv[b, kh] += p.T @ do[b, h, rows]
                else:
                    dk[b, kh][cols] += scale * (ds.T @ q[b, h, rows])
                    dv[b, kh][cols] += p.T @ do[b, h, rows]
    return dq, dk, dv


def count_allowed_pairs(q_pos, k_pos, mode, q_doc=None, k_doc=None, row_block=4096):
    """Number of allowed (query, key) pairs per head (the causal-effective work)."""
    q_pos = np.asarray(q_pos)
    total = 0
    for r0 in range(0, q_pos.size, row_block):
        rows = slice(r0, r0 + row_block)
        total += int(allowed_pairs(q_pos[rows], k_pos, mode,
                                   None if q_doc is None else np.asarray(q_doc)[rows], k_doc).sum())
    return total
