"""ctypes view of libringattn.so (the C ABI declared in include/ringattn.h).

The library must be built in-tree (``__graft_entry__.build()`` or
``python ring_attention_ringattn_amd/build.py``).  Loading fails loudly when it
is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.environ.get("RINGATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libringattn.so")

RA_OK, RA_ERR_INVALID, RA_ERR_UNSUPPORTED, RA_ERR_WORKSPACE, RA_ERR_HIP = 0, -1, -2, -3, -4
RA_MASK_NONE, RA_MASK_CAUSAL, RA_MASK_DOC_CAUSAL = 0, 1, 2
RA_F32, RA_BF16 = 0, 1
RA_STEP_FIRST, RA_STEP_LAST, RA_NO_SKIP = 1, 2, 4
RA_RUN_SERIAL_COPY, RA_RUN_POISON, RA_RUN_MERGE_KERNEL, RA_RUN_COPY_ENGINE, RA_RUN_ALLGATHER = 16, 32, 64, 128, 256
RA_PASS_FWD, RA_PASS_BWD = 1, 2
RA_MAX_SK = 262144
RA_FUSED_MAX_BLOCKS = 16
RA_NOALLOC_SCRATCH_BYTES = 36 << 20

# every function include/ringattn.h declares
EXPORTS = ("ringattn_step_workspace_size", "ringattn_step_fwd", "ringattn_step_fwd_noalloc",
           "ringattn_fused_workspace_size", "ringattn_fused_fwd",
           "ringattn_merge", "ringattn_bwd_preprocess",
           "ringattn_step_bwd", "ringattn_run_workspace_size", "ringattn_run", "ringattn_docs_from_cu_seqlens",
           "ringattn_last_error", "ringattn_version")


class RaProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("sq", ctypes.c_int32), ("sk", ctypes.c_int32),
                ("q_stride", ctypes.c_int64 * 3), ("kv_stride", ctypes.c_int64 * 3),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class RaRunDesc(ctypes.Structure):
    _fields_ = [("prob", RaProblem), ("n_ranks", ctypes.c_int32), ("n_emulated", ctypes.c_int32),
                ("first_rank", ctypes.c_int32), ("start_step", ctypes.c_int32), ("stop_step", ctypes.c_int32),
                ("mask_mode", ctypes.c_int32), ("pass_", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("step_events", ctypes.POINTER(ctypes.c_void_p))]


_P = ctypes.c_void_p
_I = ctypes.c_int
_PP = ctypes.POINTER(ctypes.c_void_p)
_SIG = {
    "ringattn_step_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(RaProblem)]),
    "ringattn_step_fwd": (_I, [ctypes.POINTER(RaProblem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _P,
                               ctypes.c_size_t, _P]),
    "ringattn_step_fwd_noalloc": (_I, [ctypes.POINTER(RaProblem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I,
                                       _P]),
    "ringattn_fused_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(RaProblem), _I]),
    "ringattn_fused_fwd": (_I, [ctypes.POINTER(RaProblem), _I, _P, _PP, _PP, _P, _P, _P, _PP, _P, _PP, _I, _I, _P,
                                ctypes.c_size_t, _P]),
    "ringattn_merge": (_I, [ctypes.POINTER(RaProblem), _P, _P, _P, _P, _P]),
    "ringattn_bwd_preprocess": (_I, [ctypes.POINTER(RaProblem), _P, _P, _P, _P]),
    "ringattn_step_bwd": (_I, [ctypes.POINTER(RaProblem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I,
                               _I, _P, ctypes.c_size_t, _P]),
    "ringattn_run_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(RaRunDesc)]),
    "ringattn_run": (_I, [ctypes.POINTER(RaRunDesc)] + [_PP] * 15 + [_P, ctypes.c_size_t, _P, _P]),
    "ringattn_docs_from_cu_seqlens": (_I, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "ringattn_last_error": (ctypes.c_char_p, []),
    "ringattn_version": (_I, []),
}

_lib = None


def load():
    """The loaded library (cached).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build(); "
                           "ring attention has no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIG.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class RingAttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"ringattn status {status}: {message}")
        self.status = status


def check(status):
    if status != RA_OK:
        raise RingAttnError(status, load().ringattn_last_error().decode())
    return status
