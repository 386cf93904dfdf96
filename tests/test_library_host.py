"""The C ABI on the host: the library loads, exports what include/ringattn.h declares,
and its pure-host validation rejects bad arguments with the documented status and
without touching any output.  No kernel is launched here (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

from ring_attention_ringattn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ringattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ringattn_\w+)\s*\(", text, flags=re.M)))


def test_header_exports_match_library():
    names = declared_functions()
    assert len(names) == 13, names
    assert sorted(_lib.EXPORTS) == names
    lib = _lib.load()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.ringattn_version() == 2


def _problem(**kw):
    """A valid bf16 problem; dense strides follow the sizes unless given."""
    p = _lib.RaProblem()
    p.batch, p.hq, p.hkv, p.head_dim, p.sq, p.sk = 1, 4, 2, 128, 256, 256
    p.dtype, p.softmax_scale = _lib.RA_BF16, 0.0
    for k, v in kw.items():
        if k not in ("q_stride", "kv_stride"):
            setattr(p, k, v)
    sq, sk, d = max(p.sq, 1), max(p.sk, 1), p.head_dim
    p.q_stride[:] = kw.get("q_stride", (p.hq * sq * d, sq * d, d))
    p.kv_stride[:] = kw.get("kv_stride", (p.hkv * sk * d, sk * d, d))
    return p


class Host:
    """Host buffers standing in for device pointers: validation must reject before touching them."""

    def __init__(self):
        self.bufs = {n: np.full(64, 7.0, dtype=np.float32) for n in
                     ("q", "k", "v", "o", "lse", "out", "qp", "kp", "qd", "kd", "ws", "do", "delta", "dq", "dk", "dv")}

    def p(self, n, off=0):
        return ctypes.c_void_p(self.bufs[n].ctypes.data + off)

    def untouched(self):
        return all(np.all(b == 7.0) for b in self.bufs.values())


def step_fwd(h, p, mask=1, flags=0, ws_bytes=1 << 20, **ptr):
    args = dict(q=h.p("q"), k=h.p("k"), v=h.p("v"), o=h.p("o"), lse=h.p("lse"), out=h.p("out"), qp=h.p("qp"),
                kp=h.p("kp"), qd=None, kd=None, ws=h.p("ws"))
    args.update(ptr)
    return _lib.load().ringattn_step_fwd(ctypes.byref(p) if p is not None else None, args["q"], args["k"],
                                         args["v"], args["o"], args["lse"], args["out"], args["qp"], args["kp"],
                                         args["qd"], args["kd"], mask, flags, args["ws"], ws_bytes, None)


CASES = [
    ("null problem", None, {}, {}, _lib.RA_ERR_INVALID),
    ("hq not a multiple of hkv", _problem(hq=3), {}, {}, _lib.RA_ERR_INVALID),
    ("head_dim 96", _problem(head_dim=96), {}, {}, _lib.RA_ERR_UNSUPPORTED),
    ("dtype 7", _problem(dtype=7), {}, {}, _lib.RA_ERR_UNSUPPORTED),
    ("negative sq", _problem(sq=-1), {}, {}, _lib.RA_ERR_INVALID),
    ("zero batch", _problem(batch=0), {}, {}, _lib.RA_ERR_INVALID),
    ("sk above the cap", _problem(sk=_lib.RA_MAX_SK + 1), {}, {}, _lib.RA_ERR_UNSUPPORTED),
    ("stride not a multiple of 8", _problem(q_stride=(4 * 256 * 128, 256 * 128, 132)), {}, {}, _lib.RA_ERR_INVALID),
    ("overlapping q rows", _problem(q_stride=(4 * 256 * 128, 256 * 128, 64)), {}, {}, _lib.RA_ERR_INVALID),
    ("kv token stride of 8 Mi elements", _problem(kv_stride=(1 << 40, 1 << 35, 8 << 20)), {}, {},
     _lib.RA_ERR_UNSUPPORTED),
    ("q token stride of 8 Mi elements", _problem(q_stride=(1 << 40, 1 << 35, 8 << 20)), {}, {},
     _lib.RA_ERR_UNSUPPORTED),
    ("negative scale", _problem(softmax_scale=-1.0), {}, {}, _lib.RA_ERR_INVALID),
    ("nan scale", _problem(softmax_scale=float("nan")), {}, {}, _lib.RA_ERR_INVALID),
    ("mask mode 3", _problem(), {"mask": 3}, {}, _lib.RA_ERR_UNSUPPORTED),
    ("doc mask without docs", _problem(), {"mask": 2}, {}, _lib.RA_ERR_INVALID),
    ("unknown flag", _problem(), {"flags": 1 << 9}, {}, _lib.RA_ERR_INVALID),
    ("null q", _problem(), {}, {"q": None}, _lib.RA_ERR_INVALID),
    ("misaligned k", _problem(), {}, {"k": "misaligned"}, _lib.RA_ERR_INVALID),
    ("null lse", _problem(), {}, {"lse": None}, _lib.RA_ERR_INVALID),
    ("workspace too small", _problem(), {"ws_bytes": 16}, {}, _lib.RA_ERR_WORKSPACE),
]


@pytest.mark.parametrize("name,p,kw,ptr,status", CASES, ids=[c[0] for c in CASES])
def test_step_fwd_validation(name, p, kw, ptr, status):
    h = Host()
    ptr = {k: (h.p(k, 2) if v == "misaligned" else v) for k, v in ptr.items()}
    rc = step_fwd(h, p, **kw, **ptr)
    assert rc == status, _lib.load().ringattn_last_error()
    assert _lib.load().ringattn_last_error()
    assert h.untouched()


def fused_fwd(h, p, n_blocks=2, mask=1, flags=0, ws_bytes=1 << 20, **ptr):
    pp = ctypes.POINTER(ctypes.c_void_p)
    arrs = []

    def arr(name, n):
        if name is None:
            return None
        a = (ctypes.c_void_p * max(n, 1))(*[h.bufs[name].ctypes.data] * max(n, 1))
        arrs.append(a)
        return ctypes.cast(a, pp)
    args = dict(q=h.p("q"), k=arr("k", n_blocks), v=arr("v", n_blocks), lse=h.p("lse"), out=h.p("out"),
                qp=h.p("qp"), kp=arr("kp", n_blocks), qd=None, kd=None, ws=h.p("ws"))
    args.update(ptr)
    return _lib.load().ringattn_fused_fwd(ctypes.byref(p), n_blocks, args["q"], args["k"], args["v"], args["lse"],
                                          args["out"], args["qp"], args["kp"], args["qd"], args["kd"], mask, flags,
                                          args["ws"], ws_bytes, None)


FUSED_CASES = [
    ("no blocks", _problem(), {"n_blocks": 0}, {}, _lib.RA_ERR_INVALID),
    ("too many blocks", _problem(), {"n_blocks": _lib.RA_FUSED_MAX_BLOCKS + 1}, {}, _lib.RA_ERR_INVALID),
    ("fp32 problem", _problem(dtype=_lib.RA_F32), {}, {}, _lib.RA_ERR_UNSUPPORTED),
    ("step flag", _problem(), {"flags": _lib.RA_STEP_FIRST}, {}, _lib.RA_ERR_INVALID),
    ("null block array", _problem(), {}, {"k": None}, _lib.RA_ERR_INVALID),
    ("null out", _problem(), {}, {"out": None}, _lib.RA_ERR_INVALID),
    ("doc mask without docs", _problem(), {"mask": 2}, {}, _lib.RA_ERR_INVALID),
    ("workspace too small", _problem(), {"ws_bytes": 16}, {}, _lib.RA_ERR_WORKSPACE),
]


@pytest.mark.parametrize("name,p,kw,ptr,status", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_fwd_validation(name, p, kw, ptr, status):
    h = Host()
    rc = fused_fwd(h, p, **kw, **ptr)
    assert rc == status, _lib.load().ringattn_last_error()
    assert _lib.load().ringattn_last_error()
    assert h.untouched()


def test_fused_workspace_size():
    lib = _lib.load()
    p = _problem(sq=1000, sk=130)
    one = lib.ringattn_fused_workspace_size(ctypes.byref(p), 1)
    four = lib.ringattn_fused_workspace_size(ctypes.byref(p), 4)
    # per block: a tile table of 3 tiles (256-aligned) and the bf16 transposed values,
    # 1 batch x 2 kv heads x 128 dims x 192 keys (130 rounded up to whole 64-key tiles)
    assert one >= (16 + 3) * 16 and four - one == 3 * (256 + 1 * 2 * 128 * 192 * 2)
    p32 = _problem(sq=1000, sk=130, dtype=_lib.RA_F32)
    assert lib.ringattn_fused_workspace_size(ctypes.byref(p32), 4) - \
        lib.ringattn_fused_workspace_size(ctypes.byref(p32), 1) == 3 * 256
    assert lib.ringattn_fused_workspace_size(ctypes.byref(p), 0) == 0
    assert lib.ringattn_fused_workspace_size(ctypes.byref(p), _lib.RA_FUSED_MAX_BLOCKS + 1) == 0


def test_empty_query_shard_is_a_no_op():
    h = Host()
    assert step_fwd(h, _problem(sq=0)) == _lib.RA_OK
    assert h.untouched()


def test_workspace_size_queries():
    lib = _lib.load()
    p = _problem(sq=1000, sk=130)
    n = lib.ringattn_step_workspace_size(ctypes.byref(p))
    assert n >= (16 + 3) * 16 and n % 256 == 0
    assert n >= 1 * 2 * 128 * 192 * 2     # room for the transposed value block of the bf16 forward
    assert lib.ringattn_step_workspace_size(ctypes.byref(_problem(head_dim=96))) == 0
    d = _lib.RaRunDesc()
    d.prob = _problem(sk=1024)
    d.n_ranks, d.n_emulated, d.mask_mode, d.pass_ = 8, 1, 1, _lib.RA_PASS_FWD
    ws = lib.ringattn_run_workspace_size(ctypes.byref(d))
    blk = 1 * 2 * 1024 * 128 * 2
    assert ws >= 2 * 2 * blk            # two staging slots of K and V
    d.n_emulated = 9
    assert lib.ringattn_run_workspace_size(ctypes.byref(d)) == 0


def _run(h, d, **arrays):
    lib = _lib.load()
    pp = ctypes.POINTER(ctypes.c_void_p)

    def arr(name, n):
        a = (ctypes.c_void_p * n)(*[h.bufs[name].ctypes.data] * n)
        arr.keep.append(a)
        return ctypes.cast(a, pp)
    arr.keep = []
    n, r = d.n_ranks, max(d.n_emulated, 1)
    A = dict(q=arr("q", r), k=arr("k", n), v=arr("v", n), o=arr("o", r), lse=arr("lse", r), out=arr("out", r),
             qp=arr("qp", r), kp=arr("kp", n), qd=None, kd=None, do=None, delta=None, dq=None, dk=None, dv=None)
    A.update(arrays)
    return lib.ringattn_run(ctypes.byref(d), A["q"], A["k"], A["v"], A["o"], A["lse"], A["out"], A["qp"], A["kp"],
                            A["qd"], A["kd"], A["do"], A["delta"], A["dq"], A["dk"], A["dv"], h.p("ws"), 1 << 30,
                            None, None)


@pytest.mark.parametrize("field,value,status", [
    ("n_emulated", 9, _lib.RA_ERR_INVALID), ("n_ranks", 0, _lib.RA_ERR_INVALID),
    ("start_step", 8, _lib.RA_ERR_INVALID), ("stop_step", -1, _lib.RA_ERR_INVALID),
    ("pass_", 3, _lib.RA_ERR_INVALID), ("first_rank", 8, _lib.RA_ERR_INVALID),
    ("flags", 1 << 12, _lib.RA_ERR_INVALID), ("mask_mode", 5, _lib.RA_ERR_UNSUPPORTED),
])
def test_run_validation(field, value, status):
    h = Host()
    d = _lib.RaRunDesc()
    d.prob = _problem()
    d.n_ranks, d.n_emulated, d.mask_mode, d.pass_ = 8, 1, 1, _lib.RA_PASS_FWD
    setattr(d, field, value)
    assert _run(h, d) == status, _lib.load().ringattn_last_error()
    assert h.untouched()


def test_run_allgather_mode_validation():
    h = Host()
    d = _lib.RaRunDesc()
    d.prob = _problem()
    d.n_ranks, d.n_emulated, d.mask_mode, d.pass_ = 8, 1, 1, _lib.RA_PASS_FWD
    d.flags = _lib.RA_RUN_ALLGATHER
    d.pass_ = _lib.RA_PASS_BWD
    assert _run(h, d) == _lib.RA_ERR_INVALID                    # forward-pass mode only
    d.pass_ = _lib.RA_PASS_FWD
    d.start_step = 1
    assert _run(h, d) == _lib.RA_ERR_INVALID                    # the whole ring only
    d.start_step = 0
    d.prob = _problem(dtype=_lib.RA_F32)
    assert _run(h, d) == _lib.RA_ERR_UNSUPPORTED                # bf16 only
    d.prob = _problem()
    d.n_ranks = _lib.RA_FUSED_MAX_BLOCKS + 1
    assert _run(h, d) == _lib.RA_ERR_UNSUPPORTED                # at most 16 resident blocks
    d.n_ranks = 8
    assert _run(h, d, out=None) == _lib.RA_ERR_INVALID          # out is required (no o_acc is written)
    assert h.untouched()


def test_run_rejects_strided_blocks_and_missing_backward_buffers():
    h = Host()
    d = _lib.RaRunDesc()
    d.prob = _problem(kv_stride=(2 * 512 * 128, 512 * 128, 128))   # gaps between heads
    d.n_ranks, d.n_emulated, d.mask_mode, d.pass_ = 4, 1, 1, _lib.RA_PASS_FWD
    assert _run(h, d) == _lib.RA_ERR_INVALID
    d.prob = _problem()
    d.pass_ = _lib.RA_PASS_BWD
    assert _run(h, d) == _lib.RA_ERR_INVALID          # no d_o / delta / dq / dk / dv
    assert b"backward" in _lib.load().ringattn_last_error()
    assert h.untouched()


def test_launch_size_limits():
    """Problems whose launches would not fit one dispatch (grid work-items are 32-bit) are
    rejected with RA_ERR_UNSUPPORTED before anything is enqueued; rows are never narrowed."""
    lib = _lib.load()
    h = Host()
    # 2^27 rows of the standalone merge (one 32-lane group each): 2^32 work-items, one too many
    p = _lib.RaProblem()
    p.batch, p.hq, p.hkv, p.head_dim, p.sq, p.dtype = 1, 32, 32, 128, 1 << 22, _lib.RA_F32
    assert lib.ringattn_merge(ctypes.byref(p), h.p("o"), h.p("lse"), h.p("dq"), h.p("delta"), None) \
        == _lib.RA_ERR_UNSUPPORTED
    assert b"merge" in lib.ringattn_last_error()
    # beyond 2^31 rows the count would also wrap a 32-bit int: still rejected, not launched
    p.batch, p.hq, p.sq = 4, 64, 1 << 24
    assert lib.ringattn_merge(ctypes.byref(p), h.p("o"), h.p("lse"), h.p("dq"), h.p("delta"), None) \
        == _lib.RA_ERR_UNSUPPORTED
    # just inside the limit the merge passes validation (then fails on the misaligned pointer)
    p.batch, p.hq, p.sq = 1, 32, (1 << 22) - 1
    assert lib.ringattn_merge(ctypes.byref(p), h.p("o", 2), h.p("lse"), h.p("dq"), h.p("delta"), None) \
        == _lib.RA_ERR_INVALID
    # a step or ring whose forward, backward or merge grid would overflow
    big = _problem(batch=64, hq=64, hkv=8, sq=1 << 20, sk=1024)
    assert step_fwd(h, big) == _lib.RA_ERR_UNSUPPORTED
    assert lib.ringattn_step_workspace_size(ctypes.byref(big)) == 0
    d = _lib.RaRunDesc()
    d.prob = big
    d.n_ranks, d.n_emulated, d.mask_mode, d.pass_, d.flags = 8, 1, 1, _lib.RA_PASS_FWD, _lib.RA_RUN_MERGE_KERNEL
    assert _run(h, d) == _lib.RA_ERR_UNSUPPORTED
    # fp32 kernels run one wave per row: 2^26 rows is one dispatch too many
    assert step_fwd(h, _problem(dtype=_lib.RA_F32, hq=64, hkv=64, sq=1 << 20)) == _lib.RA_ERR_UNSUPPORTED
    assert h.untouched()


def test_noalloc_step_rejects_what_its_scratch_cannot_hold():
    """ringattn_step_fwd_noalloc validates exactly like ringattn_step_fwd, and a problem whose
    tables and transposed value block exceed the scratch array is RA_ERR_UNSUPPORTED: all of it
    host code, before any HIP call, outputs untouched."""
    lib = _lib.load()
    h = Host()

    def call(p, **ptr):
        a = dict(q=h.p("q"), k=h.p("k"), v=h.p("v"), o=h.p("o"), lse=h.p("lse"), out=h.p("out"), qp=h.p("qp"),
                 kp=h.p("kp"))
        a.update(ptr)
        return lib.ringattn_step_fwd_noalloc(ctypes.byref(p), a["q"], a["k"], a["v"], a["o"], a["lse"], a["out"],
                                             a["qp"], a["kp"], None, None, 1, 0, None)
    # 32768-key blocks of 8 kv heads at D = 128: 64 MiB of transposed values
    big = _problem(hq=32, hkv=8, sq=32768, sk=32768)
    assert lib.ringattn_step_workspace_size(ctypes.byref(big)) > _lib.RA_NOALLOC_SCRATCH_BYTES
    assert call(big) == _lib.RA_ERR_UNSUPPORTED
    assert b"scratch" in lib.ringattn_last_error()
    # the 16384-key blocks of the 131072-token share fit
    fits = _problem(hq=32, hkv=8, sq=16384, sk=16384)
    assert lib.ringattn_step_workspace_size(ctypes.byref(fits)) <= _lib.RA_NOALLOC_SCRATCH_BYTES
    assert call(fits, q=None) == _lib.RA_ERR_INVALID          # the step's own checks come first
    assert call(_problem(head_dim=96)) == _lib.RA_ERR_UNSUPPORTED
    assert call(_problem(), kp=h.p("kp", 2)) == _lib.RA_ERR_INVALID
    assert call(_problem(sq=0)) == _lib.RA_OK                 # empty shard: nothing to do
    assert h.untouched()
