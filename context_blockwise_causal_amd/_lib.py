"""ctypes binding of libringattn (include/ra.h): argument marshalling only.

The library is loaded from this package directory; if it is missing the import of the
binding fails loudly with instructions to build it.  There is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libringattn.so")

RA_OK, RA_ERR_INVALID, RA_ERR_UNSUPPORTED, RA_ERR_DEVICE, RA_ERR_WORKSPACE = range(5)
RA_F32, RA_BF16 = 0, 1
RA_CONTIGUOUS, RA_ZIGZAG = 0, 1
RA_MASK_FULL, RA_MASK_DIAG, RA_MASK_SKIP = 0, 1, 2
RA_A2A_SEQ_PACK, RA_A2A_HEAD_UNPACK, RA_A2A_HEAD_PACK, RA_A2A_SEQ_UNPACK = 0, 1, 2, 3
RA_NOALLOC_SCRATCH_BYTES = 64 << 20  # size of the static scratch of ra_chunk_bwd_ds_noalloc
RA_DEBUG_POISON_SLOTS, RA_DEBUG_ROCTX = 1, 2  # ra_set_debug flags


class ra_problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64),
                ("heads_q", ctypes.c_int64), ("heads_kv", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("cp_size", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("window", ctypes.c_int64), ("attn_chunk", ctypes.c_int64)]


class ra_pair(ctypes.Structure):
    _fields_ = [("q_row0", ctypes.c_int64), ("kv_row0", ctypes.c_int64),
                ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64),
                ("mask", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("q_pos0", ctypes.c_int64), ("kv_pos0", ctypes.c_int64)]


class RAError(RuntimeError):
    def __init__(self, func, status, msg):
        super().__init__(f"{func}: {status_str(status)}: {msg}")
        self.status = status


class RAValueError(ValueError):
    def __init__(self, func, status, msg):
        super().__init__(f"{func}: {status_str(status)}: {msg}")
        self.status = status


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_PROB = ctypes.POINTER(ra_problem)
_PAIRS = ctypes.POINTER(ra_pair)
_FP = ctypes.c_void_p  # float* passed as raw device addresses

# name -> argtypes (restype is ra_status = int for all but the few listed below)
SIGNATURES = {
    "ra_validate": [_PROB, _I32],
    "ra_plan_step": [_PROB, _I32, _I32, ctypes.POINTER(_I32), _PAIRS, ctypes.POINTER(_I32)],
    "ra_workspace_size": [_PROB, _I32, ctypes.POINTER(ctypes.c_size_t)],
    "ra_create": [_I32, ctypes.POINTER(_P)],
    "ra_set_debug": [_P, ctypes.c_uint32],
    "ra_layout_gather": [_P, _PROB, _I32, _I32, _I64, _P, _P, _P],
    "ra_layout_scatter": [_P, _PROB, _I32, _I32, _I64, _P, _P, _P],
    "ra_ulysses_reshard": [_P, _PROB, _I32, _I64, _P, _P, _P],
    "ra_stage_kv": [_P, _PROB, _I32, _P, _P, _P, _P],
    "ra_state_init": [_P, _PROB, _I64, _FP, _FP, _FP, _P],
    "ra_chunk_fwd": [_P, _PROB, _P, _I64, _P, _P, _I64, _PAIRS, _I32, _FP, _FP, _FP, _P],
    "ra_lse_merge": [_P, _PROB, _I64, _FP, _FP, _FP, _FP, _FP, _P],
    "ra_fwd_finalize": [_P, _PROB, _I64, _FP, _FP, _FP, _P, _FP, _P],
    "ra_bwd_preprocess": [_P, _PROB, _I64, _P, _P, _FP, _P],
    "ra_chunk_bwd": [_P, _PROB, _P, _P, _FP, _FP, _I64, _P, _P, _I64, _PAIRS, _I32, _FP, _FP,
                     _FP, _P],
    "ra_chunk_bwd_ds_size": [_PROB, _I64, _I64, _PAIRS, _I32, ctypes.POINTER(ctypes.c_size_t)],
    "ra_chunk_bwd_ds": [_P, _PROB, _P, _P, _FP, _FP, _I64, _P, _P, _I64, _PAIRS, _I32, _FP, _FP,
                        _FP, _P, ctypes.c_size_t, _P],
    "ra_chunk_bwd_ds_noalloc": [_P, _PROB, _P, _P, _FP, _FP, _I64, _P, _P, _I64, _PAIRS, _I32, _FP, _FP,
                                _FP, _P],
    "ra_cast_from_f32": [_P, _PROB, _I64, _FP, _P, _P],
    "ra_rank_view_fwd": [_P, _PROB, _I32, _P, _P, _P, _P, _FP, _P, ctypes.c_size_t, _P, _P],
    "ra_rank_view_fwd_split": [_P, _PROB, _I32, _P, _P, _P, _P, _FP, _P, ctypes.c_size_t, _P, _P],
    "ra_rank_view_bwd": [_P, _PROB, _I32, _P, _P, _P, _P, _FP, _P, _P, _P, _P, _P,
                         ctypes.c_size_t, _P, _P],
}
OTHER = {
    "ra_version": ([], ctypes.c_char_p),
    "ra_status_str": ([_I32], ctypes.c_char_p),
    "ra_last_error": ([], ctypes.c_char_p),
    "ra_destroy": ([_P], None),
}

_lib = None


def load():
    """Loads libringattn.so (once).  Raises RuntimeError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m "
                           "context_blockwise_causal_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in SIGNATURES.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    for name, (args, res) in OTHER.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().ra_status_str(status).decode()


def last_error() -> str:
    return load().ra_last_error().decode()


def check(func: str, status: int):
    if status == RA_OK:
        return
    msg = last_error()
    if status in (RA_ERR_INVALID, RA_ERR_UNSUPPORTED, RA_ERR_WORKSPACE):
        raise RAValueError(func, status, msg)
    raise RAError(func, status, msg)


def call(func: str, *args):
    """Calls an ra_status-returning entry point and raises on failure."""
    check(func, getattr(load(), func)(*args))


def problem(batch, seq_len, heads_q, heads_kv, head_dim, cp_size, layout, dtype, scale=0.0, window=0,
            attn_chunk=0):
    lay = {"contiguous": RA_CONTIGUOUS, "zigzag": RA_ZIGZAG}.get(layout, layout)
    dt = {"f32": RA_F32, "bf16": RA_BF16}.get(dtype, dtype)
    return ra_problem(batch, seq_len, heads_q, heads_kv, head_dim, cp_size, lay, dt, scale, window,
                      attn_chunk)


def pairs_array(pairs):
    """[(q_row0, kv_row0, q_len, kv_len, mask[, q_pos0, kv_pos0]), ...] -> ctypes array of
    ra_pair (positions default to 0; they matter only for window / attention-chunk masks)."""
    arr = (ra_pair * max(1, len(pairs)))()
    for i, p in enumerate(pairs):
        q0, k0, ql, kl, mask = p[:5]
        qp, kp = (p[5], p[6]) if len(p) > 5 else (0, 0)
        arr[i] = ra_pair(q0, k0, ql, kl, mask, 0, qp, kp)
    return arr
