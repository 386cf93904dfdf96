"""Ring attention's per-device hot path on MI355X: a thin binding over libringattn.

Every function here has the name of the C entry point it calls (see
include/ringattn.h) and only marshals arguments: torch tensors become device
pointers and strides, torch streams become hipStream_t handles, and the
workspace is a torch byte tensor when the caller does not pass one.  All
arithmetic runs in the library's HIP kernels; when the library is missing,
the first call raises.

Layouts: q, d_o, out are [B, Hq, Sq, D] views (any batch/head/token strides,
D contiguous), k, v are [B, Hkv, Sk, D] views; o_acc, dq are dense fp32
[B, Hq, Sq, D]; dk, dv dense fp32 [B, Hkv, Sk, D]; lse, delta dense fp32
[B, Hq, Sq]; positions and documents are int32 [S] device tensors.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import (RA_BF16, RA_F32, RA_MASK_CAUSAL, RA_MASK_DOC_CAUSAL, RA_MASK_NONE, RA_MAX_SK, RA_NO_SKIP,
                   RA_PASS_BWD, RA_PASS_FWD, RA_RUN_ALLGATHER, RA_RUN_COPY_ENGINE, RA_RUN_MERGE_KERNEL,
                   RA_RUN_POISON, RA_RUN_SERIAL_COPY, RA_STEP_FIRST, RA_STEP_LAST, RA_FUSED_MAX_BLOCKS,
                   RA_NOALLOC_SCRATCH_BYTES, RingAttnError)
from . import sharding

__all__ = ["ringattn_step_workspace_size", "ringattn_step_fwd", "ringattn_step_fwd_noalloc",
           "ringattn_fused_workspace_size",
           "ringattn_fused_fwd", "ringattn_merge", "ringattn_bwd_preprocess",
           "ringattn_step_bwd", "ringattn_run_workspace_size", "ringattn_run", "ringattn_docs_from_cu_seqlens",
           "ringattn_last_error", "ringattn_version", "make_problem", "RingAttnError", "sharding",
           "RA_MASK_NONE", "RA_MASK_CAUSAL", "RA_MASK_DOC_CAUSAL", "RA_STEP_FIRST", "RA_STEP_LAST", "RA_NO_SKIP",
           "RA_RUN_SERIAL_COPY", "RA_RUN_POISON", "RA_RUN_MERGE_KERNEL", "RA_RUN_COPY_ENGINE", "RA_RUN_ALLGATHER",
           "RA_FUSED_MAX_BLOCKS", "RA_PASS_FWD",
           "RA_PASS_BWD",
           "RA_F32", "RA_BF16", "RA_MAX_SK", "RA_NOALLOC_SCRATCH_BYTES"]

_DTYPES = {torch.float32: RA_F32, torch.bfloat16: RA_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def make_problem(q: torch.Tensor, k: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                 sk: Optional[int] = None, hkv: Optional[int] = None) -> _lib.RaProblem:
    """ra_problem for a query view q [B,Hq,Sq,D] and a key view k [B,Hkv,Sk,D]."""
    if q.dim() != 4:
        raise ValueError("q must be a [B, Hq, Sq, D] view")
    if q.stride(3) != 1:
        raise ValueError("the head dimension of q must be contiguous")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    p = _lib.RaProblem()
    p.batch, p.hq, p.sq, p.head_dim = q.shape[0], q.shape[1], q.shape[2], q.shape[3]
    p.q_stride[:] = q.stride()[:3]
    if k is not None:
        if k.dim() != 4 or k.stride(3) != 1:
            raise ValueError("k must be a [B, Hkv, Sk, D] view with contiguous head dimension")
        if k.dtype != q.dtype:
            raise ValueError("q and k must share a dtype")
        p.hkv, p.sk = k.shape[1], k.shape[2]
        p.kv_stride[:] = k.stride()[:3]
    else:
        p.hkv = hkv if hkv is not None else q.shape[1]
        p.sk = sk if sk is not None else 0
        p.kv_stride[:] = q.stride()[:3]
    p.dtype = _DTYPES[q.dtype]
    p.softmax_scale = softmax_scale
    return p


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def ringattn_version() -> int:
    return _lib.load().ringattn_version()


def ringattn_last_error() -> str:
    return _lib.load().ringattn_last_error().decode()


def ringattn_step_workspace_size(q: torch.Tensor, k: torch.Tensor) -> int:
    p = make_problem(q, k)
    return _lib.load().ringattn_step_workspace_size(ctypes.byref(p))


def ringattn_step_fwd(q, k_blk, v_blk, o_acc, lse, out, q_pos, kv_pos, q_doc=None, kv_doc=None,
                      mask_mode=RA_MASK_CAUSAL, flags=0, workspace=None, stream=None, softmax_scale=0.0):
    """One forward ring step into the running (o_acc, lse); see ringattn_step_fwd in the header."""
    lib = _lib.load()
    if v_blk.stride() != k_blk.stride() or v_blk.shape != k_blk.shape:
        raise ValueError("k_blk and v_blk must have the same shape and strides")
    if out is not None and out.stride() != q.stride():
        raise ValueError("out must have the strides of q")
    p = make_problem(q, k_blk, softmax_scale)
    need = lib.ringattn_step_workspace_size(ctypes.byref(p))
    ws = _workspace(need, q.device, workspace)
    return _lib.check(lib.ringattn_step_fwd(
        ctypes.byref(p), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(o_acc), _ptr(lse), _ptr(out), _ptr(q_pos),
        _ptr(kv_pos), _ptr(q_doc), _ptr(kv_doc), mask_mode, flags, _ptr(ws), ws.numel(), _stream(stream)))


def ringattn_step_fwd_noalloc(q, k_blk, v_blk, o_acc, lse, out, q_pos, kv_pos, q_doc=None, kv_doc=None,
                              mask_mode=RA_MASK_CAUSAL, flags=0, stream=None, softmax_scale=0.0):
    """ringattn_step_fwd with the library's own device scratch instead of a workspace (no
    allocation on any path: not here, not in the library); see the header for its limit."""
    lib = _lib.load()
    if v_blk.stride() != k_blk.stride() or v_blk.shape != k_blk.shape:
        raise ValueError("k_blk and v_blk must have the same shape and strides")
    if out is not None and out.stride() != q.stride():
        raise ValueError("out must have the strides of q")
    p = make_problem(q, k_blk, softmax_scale)
    return _lib.check(lib.ringattn_step_fwd_noalloc(
        ctypes.byref(p), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(o_acc), _ptr(lse), _ptr(out), _ptr(q_pos),
        _ptr(kv_pos), _ptr(q_doc), _ptr(kv_doc), mask_mode, flags, _stream(stream)))


def ringattn_fused_workspace_size(q: torch.Tensor, k: torch.Tensor, n_blocks: int) -> int:
    p = make_problem(q, k)
    return _lib.load().ringattn_fused_workspace_size(ctypes.byref(p), n_blocks)


def _c_ptrs(ts):
    """ctypes array of the tensors' device pointers (kept alive by the caller for the call)."""
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def ringattn_fused_fwd(q, k_blocks, v_blocks, lse, out, q_pos, kv_pos, q_doc=None, kv_doc=None,
                       mask_mode=RA_MASK_CAUSAL, flags=0, workspace=None, stream=None, softmax_scale=0.0):
    """Attention of q over every resident block in one launch (all-gather mode); see
    ringattn_fused_fwd in the header.  k_blocks, v_blocks, kv_pos (and kv_doc) are lists."""
    lib = _lib.load()
    n = len(k_blocks)
    if len(v_blocks) != n or len(kv_pos) != n or (kv_doc is not None and len(kv_doc) != n):
        raise ValueError("k_blocks, v_blocks, kv_pos (and kv_doc) must have one entry per block")
    for kb, vb in zip(k_blocks, v_blocks):
        if kb.stride() != k_blocks[0].stride() or kb.shape != k_blocks[0].shape or vb.stride() != kb.stride() \
                or vb.shape != kb.shape:
            raise ValueError("every K and V block must have one shape and one set of strides")
    if out.stride() != q.stride():
        raise ValueError("out must have the strides of q")
    p = make_problem(q, k_blocks[0], softmax_scale)
    need = lib.ringattn_fused_workspace_size(ctypes.byref(p), n)
    ws = _workspace(need, q.device, workspace)
    kd = _c_ptrs(kv_doc) if kv_doc is not None else None
    return _lib.check(lib.ringattn_fused_fwd(
        ctypes.byref(p), n, _ptr(q), _c_ptrs(k_blocks), _c_ptrs(v_blocks), _ptr(lse), _ptr(out), _ptr(q_pos),
        _c_ptrs(kv_pos), _ptr(q_doc), kd, mask_mode, flags, _ptr(ws), ws.numel(), _stream(stream)))


def ringattn_merge(o_a, lse_a, o_b, lse_b, stream=None):
    """(o_b, lse_b) <- (o_a, lse_a) (+) (o_b, lse_b), in place."""
    lib = _lib.load()
    if o_a.shape != o_b.shape or not (o_a.is_contiguous() and o_b.is_contiguous()):
        raise ValueError("o_a and o_b must be dense tensors of one shape")
    p = _lib.RaProblem()
    p.batch, p.hq, p.sq, p.head_dim = o_b.shape
    p.hkv, p.dtype = p.hq, RA_F32
    return _lib.check(lib.ringattn_merge(ctypes.byref(p), _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b),
                                         _stream(stream)))


def ringattn_bwd_preprocess(out, d_o, delta, stream=None):
    """delta = rowsum(d_o * out)."""
    lib = _lib.load()
    if d_o.stride() != out.stride():
        raise ValueError("out and d_o must have the same strides")
    p = make_problem(out)
    return _lib.check(lib.ringattn_bwd_preprocess(ctypes.byref(p), _ptr(out), _ptr(d_o), _ptr(delta),
                                                  _stream(stream)))


def ringattn_step_bwd(q, k_blk, v_blk, d_o, lse, delta, dq, dk, dv, q_pos, kv_pos, q_doc=None, kv_doc=None,
                      mask_mode=RA_MASK_CAUSAL, flags=0, workspace=None, stream=None, softmax_scale=0.0):
    """Gradient contributions of one block, accumulated into dq, dk, dv."""
    lib = _lib.load()
    if v_blk.stride() != k_blk.stride() or d_o.stride() != q.stride():
        raise ValueError("v_blk must have k_blk's strides and d_o q's strides")
    p = make_problem(q, k_blk, softmax_scale)
    need = lib.ringattn_step_workspace_size(ctypes.byref(p))
    ws = _workspace(need, q.device, workspace)
    return _lib.check(lib.ringattn_step_bwd(
        ctypes.byref(p), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(d_o), _ptr(lse), _ptr(delta), _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(q_pos), _ptr(kv_pos), _ptr(q_doc), _ptr(kv_doc), mask_mode, flags, _ptr(ws),
        ws.numel(), _stream(stream)))


def _run_desc(q, k, n_ranks, n_emulated, first_rank, start_step, stop_step, mask_mode, pass_, flags,
              softmax_scale, step_events=None):
    d = _lib.RaRunDesc()
    if step_events is not None:
        arr = (ctypes.c_void_p * len(step_events))(*step_events)
        d._events_keepalive = arr
        d.step_events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    d.prob = make_problem(q, k, softmax_scale)
    d.n_ranks, d.n_emulated, d.first_rank = n_ranks, n_emulated, first_rank
    d.start_step, d.stop_step, d.mask_mode, d.pass_, d.flags = start_step, stop_step, mask_mode, pass_, flags
    return d


def ringattn_run_workspace_size(q, k, n_ranks, n_emulated, pass_=RA_PASS_FWD, flags=0, mask_mode=RA_MASK_CAUSAL):
    d = _run_desc(q, k, n_ranks, n_emulated, 0, 0, 0, mask_mode, pass_, flags, 0.0)
    return _lib.load().ringattn_run_workspace_size(ctypes.byref(d))


def _ptr_array(ts: Optional[Sequence[Optional[torch.Tensor]]]):
    if ts is None:
        return None
    arr = (ctypes.c_void_p * len(ts))(*[None if t is None else t.data_ptr() for t in ts])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), arr


def ringattn_run(q: Sequence[torch.Tensor], k_home: Sequence[torch.Tensor], v_home: Sequence[torch.Tensor],
                 q_pos, kv_pos, *, o_acc=None, lse=None, out=None, q_doc=None, kv_doc=None, d_o=None, delta=None,
                 dq=None, dk=None, dv=None, first_rank=0, start_step=0, stop_step=0, mask_mode=RA_MASK_CAUSAL,
                 pass_=RA_PASS_FWD, flags=0, workspace=None, compute_stream=None, copy_stream=None,
                 softmax_scale=0.0, step_events=None):
    """N virtual ring steps for len(q) emulated ranks over len(k_home) blocks (see ringattn_run).

    ``step_events``: optional list of 2N raw hipEvent_t handles (ints) recorded around each step.
    """
    lib = _lib.load()
    n, r = len(k_home), len(q)
    for t in list(k_home) + list(v_home):
        if t.stride() != k_home[0].stride() or t.shape != k_home[0].shape:
            raise ValueError("every home K/V block must share shape and strides")
    for t in list(q) + list(out or []) + list(d_o or []):
        if t is not None and t.stride() != q[0].stride():
            raise ValueError("every q/out/d_o shard must share q[0]'s strides")
    d = _run_desc(q[0], k_home[0], n, r, first_rank, start_step, stop_step, mask_mode, pass_, flags, softmax_scale,
                  step_events)
    need = lib.ringattn_run_workspace_size(ctypes.byref(d))
    if need == 0:
        raise RingAttnError(_lib.RA_ERR_INVALID, ringattn_last_error())
    ws = _workspace(need, q[0].device, workspace)
    keep = []

    def arr(ts):
        if ts is None:
            return None
        a = _ptr_array(ts)
        keep.append(a[1])
        return a[0]

    cs = _stream(compute_stream)
    xs = ctypes.c_void_p(0) if copy_stream is None else _stream(copy_stream)
    return _lib.check(lib.ringattn_run(
        ctypes.byref(d), arr(q), arr(k_home), arr(v_home), arr(o_acc), arr(lse), arr(out), arr(q_pos),
        arr(kv_pos), arr(q_doc), arr(kv_doc), arr(d_o), arr(delta), arr(dq), arr(dk), arr(dv), _ptr(ws),
        ws.numel(), cs, xs))


def ringattn_docs_from_cu_seqlens(cu_seqlens: torch.Tensor, first_token: int, n_tokens: int,
                                  doc: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Document id of tokens [first_token, first_token + n_tokens) of a packed stream."""
    lib = _lib.load()
    if doc is None:
        doc = torch.empty(n_tokens, dtype=torch.int32, device=cu_seqlens.device)
    _lib.check(lib.ringattn_docs_from_cu_seqlens(_ptr(cu_seqlens), cu_seqlens.numel() - 1, first_token, n_tokens,
                                                 _ptr(doc), _stream(stream)))
    return doc
