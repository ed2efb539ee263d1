"""ctypes loader for libsegattn.so (built in-tree by ``build.py``).

There is no fallback of any kind: if the library is missing or fails to load,
importing the binding raises, naming the build command.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsegattn.so")

SEGATTN_OK = 0
SEGATTN_E_INVALID = 1
SEGATTN_E_UNSUPPORTED = 2
SEGATTN_E_RANGE = 3
SEGATTN_E_CAPACITY = 4
SEGATTN_E_WORKSPACE = 5
SEGATTN_E_DEVICE = 6

SEGATTN_BF16 = 0
SEGATTN_F32 = 1

SEGATTN_MERGE_INTO = 1
SEGATTN_ACCUMULATE = 2
SEGATTN_D_READY = 4
SEGATTN_SPLIT_KEYS = 8

SEGATTN_D2H = 0
SEGATTN_H2D = 1

SEGATTN_NOALLOC_SCRATCH_BYTES = 64 << 20

# Every symbol declared in include/segattn.h.
EXPORTS = (
    "segattn_partition",
    "segattn_partition_varlen",
    "segattn_ring_items",
    "segattn_chunk_varlen",
    "segattn_fwd_workspace",
    "segattn_fwd",
    "segattn_merge",
    "segattn_bwd_workspace",
    "segattn_bwd_preprocess",
    "segattn_offload_plan",
    "segattn_copy_rows",
    "segattn_stream_order",
    "segattn_bwd",
    "segattn_bwd_noalloc",
    "segattn_status_string",
    "segattn_last_error",
    "segattn_version",
)


class Item(ctypes.Structure):
    _fields_ = [("seq_off", ctypes.c_int64), ("q_lo", ctypes.c_int64), ("q_hi", ctypes.c_int64),
                ("k_lo", ctypes.c_int64), ("k_hi", ctypes.c_int64)]


class Shape(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class SegattnError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{_status_name(status)}: {detail}")


_lib = None


def _status_name(status):
    return lib().segattn_status_string(status).decode()


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run `python -m segmented_causal_attention_amd.build` "
                          "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER
    L.segattn_partition.argtypes = [i64, i32, P(i64)]
    L.segattn_partition_varlen.argtypes = [P(i64), i32, i64, P(Item), i32, P(i32)]
    L.segattn_ring_items.argtypes = [P(i64), i32, i64, P(Item), i32, P(i32)]
    L.segattn_chunk_varlen.argtypes = [P(i64), i32, i32, ctypes.c_double, ctypes.c_double, i64, P(Item), P(i32),
                                       i32, P(i32), P(i32), P(ctypes.c_double)]
    # item tables of the attention calls: host addresses (int) of int64 [n, 5] arrays
    L.segattn_fwd_workspace.argtypes = [P(Shape), vp, i32, P(sz)]
    L.segattn_fwd.argtypes = [P(Shape), vp, vp, vp, vp, i32, vp, i32, vp, ctypes.c_uint32, vp, sz, vp]
    L.segattn_merge.argtypes = [i64, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp]
    L.segattn_bwd_workspace.argtypes = [P(Shape), vp, i32, P(sz)]
    L.segattn_bwd_preprocess.argtypes = [P(Shape), vp, i32, vp, vp, i32, vp, sz, vp]
    L.segattn_bwd.argtypes = [P(Shape), vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, vp, i32,
                              ctypes.c_uint32, vp, sz, vp]
    L.segattn_bwd_noalloc.argtypes = [P(Shape), vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, vp, i32,
                                      ctypes.c_uint32, vp]
    f64 = ctypes.c_double
    L.segattn_offload_plan.argtypes = [P(i64), P(i64), i32, f64, P(f64), P(i64), P(f64), P(f64)]
    L.segattn_copy_rows.argtypes = [vp, i64, vp, i64, i64, i64, i32, vp]
    L.segattn_stream_order.argtypes = [vp, vp, vp]
    for name in EXPORTS:
        fn = getattr(L, name)
        if name in ("segattn_status_string", "segattn_last_error", "segattn_version"):
            fn.restype = ctypes.c_char_p
        else:
            fn.restype = ctypes.c_int
    L.segattn_status_string.argtypes = [ctypes.c_int]
    L.segattn_last_error.argtypes = []
    L.segattn_version.argtypes = []
    _lib = L
    return L


def check(status):
    if status != SEGATTN_OK:
        raise SegattnError(status, lib().segattn_last_error().decode())
    return status
