"""Python binding of libsegattn.so: argument marshalling only.

Every function has the name of the C entry point it calls
(``segattn_fwd_prepare`` prepares a repeated ``segattn_fwd``).  Device buffers are
torch tensors (torch provides device memory and the current HIP stream);
item tables are host ``numpy.int64`` arrays of shape [n, 5] with columns
(seq_off, q_lo, q_hi, k_lo, k_hi).  A nonzero status raises ``SegattnError``
carrying ``segattn_last_error()``.  Nothing here computes any part of the
attention path: all of it runs in the library's HIP kernels.
"""

from __future__ import annotations

import ctypes
import math

import numpy as np
import torch

from . import _lib
from ._lib import (SEGATTN_ACCUMULATE, SEGATTN_BF16, SEGATTN_D_READY, SEGATTN_F32,  # noqa: F401
                   SEGATTN_MERGE_INTO, SEGATTN_SPLIT_KEYS, Item, SegattnError, Shape, check, lib)

_I64P = ctypes.POINTER(ctypes.c_int64)
_ITEMP = ctypes.POINTER(Item)

_DTYPE_CODE = {torch.bfloat16: SEGATTN_BF16, torch.float32: SEGATTN_F32}
_CODE_DTYPE = {SEGATTN_BF16: torch.bfloat16, SEGATTN_F32: torch.float32}


# ------------------------------------------------------------------ helpers

def _items_arg(items):
    """(array, pointer, n) of an int64 [n, 5] item table; an array that is
    already int64, C-contiguous and [n, 5] is passed as it is."""
    if (type(items) is np.ndarray and items.dtype == np.int64 and items.ndim == 2 and items.shape[1] == 5
            and items.flags.c_contiguous):
        a = items
    else:
        a = np.ascontiguousarray(np.asarray(items, dtype=np.int64).reshape(-1, 5))
    return a, a.ctypes.data, a.shape[0]


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t, name, dtype=None):
    if type(t) is not torch.Tensor or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


_SHAPES = {}


def make_shape(q, k, scale=None):
    """segattn_shape for token-major q [T, hq, d] and k [T, hkv, d] (one
    ctypes struct per distinct shape, reused: the library only reads it)."""
    qs, ks, qd = q.shape, k.shape, q.dtype
    key = (qs, ks, qd, scale)
    sh = _SHAPES.get(key)
    if sh is None:
        if len(qs) != 3 or len(ks) != 3 or qs[0] != ks[0] or qs[2] != ks[2]:
            raise ValueError("q must be [T, hq, d] and k [T, hkv, d]")
        if qd not in _DTYPE_CODE or k.dtype != qd:
            raise TypeError("q, k, v must all be bfloat16 or all float32")
        d = qs[2]
        sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
        sh = Shape(qs[0], qs[1], ks[1], d, _DTYPE_CODE[qd], sc)
        if len(_SHAPES) < 256:
            _SHAPES[key] = sh
    return sh


def _same(t, name, shape, dtype=None, dtypes=None):
    """Raises unless t has exactly `shape` (and `dtype`, or one of `dtypes`).
    The C layer only sees pointers, so every buffer's size and element type
    is checked here, before anything is launched."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {dtypes}, got {t.dtype}")


def _check_kv(q, k, v):
    _same(v, "v", k.shape, k.dtype)


def _check_stats(q, o, lse):
    """o [T, hq, d] in bf16 or fp32; lse [hq, T] fp32."""
    _same(o, "o", q.shape, dtypes=(torch.bfloat16, torch.float32))
    _same(lse, "lse", torch.Size((q.shape[1], q.shape[0])), torch.float32)


def _workspace(nbytes, device, workspace):
    """The caller's workspace, or a new one of nbytes() bytes.  A given
    workspace is not measured here: the library checks its size (E_WORKSPACE)
    before launching anything, which saves a planning pass per call."""
    if workspace is None:
        return torch.empty(max(int(nbytes()), 16), dtype=torch.uint8, device=device)
    return workspace


# ------------------------------------------------------------------ planner

def segattn_partition(S, N):
    out = np.zeros(int(N) + 1 if int(N) >= 0 else 1, dtype=np.int64)
    check(lib().segattn_partition(int(S), int(N), out.ctypes.data_as(_I64P)))
    return out


def segattn_partition_varlen(cu_seqlens, max_slice):
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n = ctypes.c_int32(0)
    L = lib()
    st = L.segattn_partition_varlen(cu.ctypes.data_as(_I64P), len(cu) - 1, int(max_slice), None, 0,
                                    ctypes.byref(n))
    if st != _lib.SEGATTN_E_CAPACITY:
        check(st)
        if n.value == 0:
            return np.zeros((0, 5), dtype=np.int64)
    out = np.zeros((n.value, 5), dtype=np.int64)
    check(L.segattn_partition_varlen(cu.ctypes.data_as(_I64P), len(cu) - 1, int(max_slice),
                                     out.ctypes.data_as(_ITEMP), n.value, ctypes.byref(n)))
    return out


def segattn_chunk_varlen(cu_seqlens, K, alpha1, alpha2, token_cap):
    """Workload-balanced chunks of a packed batch: returns (items int64
    [n, 5], chunk index of each item int32 [n], number of chunks, final time
    threshold)."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n, nc, tt = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_double(0.0)
    L = lib()
    args = (cu.ctypes.data_as(_I64P), len(cu) - 1, int(K), float(alpha1), float(alpha2), int(token_cap))
    st = L.segattn_chunk_varlen(*args, None, None, 0, ctypes.byref(n), ctypes.byref(nc), ctypes.byref(tt))
    if st != _lib.SEGATTN_E_CAPACITY:
        check(st)
    out = np.zeros((n.value, 5), dtype=np.int64)
    owner = np.zeros(n.value, dtype=np.int32)
    check(L.segattn_chunk_varlen(*args, out.ctypes.data_as(_ITEMP),
                                 owner.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n.value, ctypes.byref(n),
                                 ctypes.byref(nc), ctypes.byref(tt)))
    return out, owner, nc.value, tt.value


def segattn_ring_items(bounds, block):
    b = np.ascontiguousarray(np.asarray(bounds, dtype=np.int64))
    n = ctypes.c_int32(0)
    L = lib()
    st = L.segattn_ring_items(b.ctypes.data_as(_I64P), len(b) - 1, int(block), None, 0, ctypes.byref(n))
    if st != _lib.SEGATTN_E_CAPACITY:
        check(st)
    out = np.zeros((n.value, 5), dtype=np.int64)
    check(L.segattn_ring_items(b.ctypes.data_as(_I64P), len(b) - 1, int(block), out.ctypes.data_as(_ITEMP),
                               n.value, ctypes.byref(n)))
    return out


# ------------------------------------------------------------------ forward

def segattn_fwd_workspace(shape, items):
    arr, p, n = _items_arg(items)
    nb = ctypes.c_size_t(0)
    check(lib().segattn_fwd_workspace(ctypes.byref(shape), p, n, ctypes.byref(nb)))
    return nb.value


def _fwd_args(q, k, v, items, scale, o, o_dtype, lse, merge_into, split_keys, workspace, stream):
    """Checked and converted arguments of one segattn_fwd call, the buffers
    they point into (kept alive with them), and (o, lse)."""
    shape = make_shape(q, k, scale)
    _check_kv(q, k, v)
    arr, p, n = _items_arg(items)
    if o is None:
        od = _CODE_DTYPE[o_dtype] if isinstance(o_dtype, int) else (o_dtype or q.dtype)
        o = torch.zeros((q.shape[0], q.shape[1], q.shape[2]), dtype=od, device=q.device)
    if lse is None:
        lse = torch.full((q.shape[1], q.shape[0]), -math.inf, dtype=torch.float32, device=q.device)
    _check_stats(q, o, lse)
    ocode = _DTYPE_CODE[o.dtype]
    ws = _workspace(lambda: segattn_fwd_workspace(shape, arr), q.device, workspace)
    flags = (SEGATTN_MERGE_INTO if merge_into else 0) | (SEGATTN_SPLIT_KEYS if split_keys else 0)
    args = (ctypes.byref(shape), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), p, n, _dev(o, "o"), ocode,
            _dev(lse, "lse", torch.float32), flags, _dev(ws, "workspace"), ws.numel() * ws.element_size(),
            _stream(stream))
    return args, (shape, q, k, v, arr, o, lse, ws), o, lse


def segattn_fwd(q, k, v, items, *, scale=None, o=None, o_dtype=None, lse=None, merge_into=False,
                split_keys=False, workspace=None, stream=None):
    """Partial attention of `items` into (o, lse); returns (o, lse).
    New outputs are allocated (o_dtype defaults to q's dtype; lse filled
    with -inf) when not given.  split_keys sets SEGATTN_SPLIT_KEYS."""
    args, _, o, lse = _fwd_args(q, k, v, items, scale, o, o_dtype, lse, merge_into, split_keys, workspace, stream)
    check(lib().segattn_fwd(*args))
    return o, lse


def segattn_fwd_prepare(q, k, v, items, *, o, lse, scale=None, merge_into=False, split_keys=False,
                        workspace=None, stream=None):
    """segattn_fwd with its arguments checked and converted once, for a call
    repeated on the same buffers (a training or serving loop with fixed
    shapes).  Returns a callable that issues the identical C call -- same
    tensors, items, flags, workspace and stream (the current stream at
    preparation when none is given) -- with no per-call Python work but the
    foreign call itself.  The callable holds references to every tensor and
    to the item table, so their memory stays valid; their contents may
    change between calls, their storage must not be replaced."""
    args, keep, _, _ = _fwd_args(q, k, v, items, scale, o, None, lse, merge_into, split_keys, workspace, stream)
    fn = lib().segattn_fwd

    def call():
        st = fn(*args)
        if st:
            check(st)

    call.buffers = keep
    return call


def segattn_merge(o_a, lse_a, o_b, lse_b, *, o_out=None, lse_out=None, rows=None, lse_stride=None,
                  stream=None):
    """Log-sum-exp merge of fp32 partials o [rows, h, d], lse [h, >= rows]."""
    if o_out is None:
        o_out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    if not isinstance(o_a, torch.Tensor) or o_a.dim() != 3:
        raise ValueError("o_a must be [rows, h, d]")
    if not isinstance(lse_a, torch.Tensor) or lse_a.dim() != 2:
        raise ValueError("lse_a must be [h, stride]")
    for t, nm in ((o_b, "o_b"), (o_out, "o_out")):
        _same(t, nm, o_a.shape, torch.float32)
    _same(o_a, "o_a", o_a.shape, torch.float32)
    r = o_a.shape[0] if rows is None else int(rows)
    stride = lse_a.stride(0) if lse_stride is None else int(lse_stride)
    if not 1 <= r <= o_a.shape[0]:
        raise ValueError(f"rows = {r} outside [1, {o_a.shape[0]}]")
    # lse operands: [h, >= rows] views with unit column stride whose rows are
    # lse_stride elements apart (a column slice of a [h, T] tensor is fine)
    for t, nm in ((lse_a, "lse_a"), (lse_b, "lse_b"), (lse_out, "lse_out")):
        if not isinstance(t, torch.Tensor) or t.dim() != 2 or t.shape[0] != o_a.shape[1] or t.shape[1] < r:
            raise ValueError(f"{nm} must be [h = {o_a.shape[1]}, >= rows = {r}]")
        if t.dtype != torch.float32:
            raise TypeError(f"{nm} must be {torch.float32}, got {t.dtype}")
        if t.stride(1) != 1 or (t.shape[0] > 1 and t.stride(0) != stride):
            raise ValueError(f"{nm} must have unit column stride and row stride lse_stride = {stride}")
    for t, nm in ((o_a, "o_a"), (o_b, "o_b"), (o_out, "o_out")):
        _dev(t, nm, torch.float32)
    for t, nm in ((lse_a, "lse_a"), (lse_b, "lse_b"), (lse_out, "lse_out")):
        if not t.is_cuda:
            raise TypeError(f"{nm} must be a float32 device tensor")
    check(lib().segattn_merge(r, o_a.shape[1], o_a.shape[2], stride, ctypes.c_void_p(o_a.data_ptr()),
                              ctypes.c_void_p(lse_a.data_ptr()), ctypes.c_void_p(o_b.data_ptr()),
                              ctypes.c_void_p(lse_b.data_ptr()), ctypes.c_void_p(o_out.data_ptr()),
                              ctypes.c_void_p(lse_out.data_ptr()), _stream(stream)))
    return o_out, lse_out


# ----------------------------------------------------------------- backward

def segattn_bwd_workspace(shape, items):
    arr, p, n = _items_arg(items)
    nb = ctypes.c_size_t(0)
    check(lib().segattn_bwd_workspace(ctypes.byref(shape), p, n, ctypes.byref(nb)))
    return nb.value


def segattn_bwd_preprocess(q, k, o, do, items, workspace, *, scale=None, stream=None):
    shape = make_shape(q, k, scale)
    _same(o, "o", q.shape, dtypes=(torch.bfloat16, torch.float32))
    _same(do, "do", q.shape, q.dtype)
    arr, p, n = _items_arg(items)
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a tensor")
    need = segattn_bwd_workspace(shape, arr)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace too small: {need} bytes needed")
    check(lib().segattn_bwd_preprocess(ctypes.byref(shape), _dev(o, "o"), _DTYPE_CODE[o.dtype], _dev(do, "do"),
                                       p, n, _dev(workspace, "workspace"), workspace.numel(), _stream(stream)))


def segattn_bwd(q, k, v, o, lse, do, items, *, scale=None, dq=None, dk=None, dv=None, g_dtype=None,
                accumulate=False, d_ready=False, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of sum(do * o); allocated (zero-filled) when
    not given, in g_dtype (default q's dtype; float32 with accumulate)."""
    shape = make_shape(q, k, scale)
    _check_kv(q, k, v)
    _check_stats(q, o, lse)
    _same(do, "do", q.shape, q.dtype)
    arr, p, n = _items_arg(items)
    gd = g_dtype or (dq.dtype if dq is not None else (torch.float32 if accumulate else q.dtype))
    if dq is None:
        dq = torch.zeros(q.shape, dtype=gd, device=q.device)
    if dk is None:
        dk = torch.zeros(k.shape, dtype=gd, device=q.device)
    if dv is None:
        dv = torch.zeros(v.shape, dtype=gd, device=q.device)
    _same(dq, "dq", q.shape, dtypes=(torch.bfloat16, torch.float32))
    _same(dk, "dk", k.shape, dq.dtype)
    _same(dv, "dv", k.shape, dq.dtype)
    if accumulate and dq.dtype != torch.float32:
        raise TypeError("accumulate=True needs float32 gradients")
    ws = _workspace(lambda: segattn_bwd_workspace(shape, arr), q.device, workspace)
    flags = (SEGATTN_ACCUMULATE if accumulate else 0) | (SEGATTN_D_READY if d_ready else 0)
    check(lib().segattn_bwd(ctypes.byref(shape), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"),
                            _DTYPE_CODE[o.dtype], _dev(lse, "lse", torch.float32), _dev(do, "do"), p, n,
                            _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"), _DTYPE_CODE[dq.dtype], flags,
                            _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream(stream)))
    return dq, dk, dv


def segattn_bwd_noalloc(q, k, v, o, lse, do, items, dq, dk, dv, *, scale=None, accumulate=False, stream=None):
    """segattn_bwd without a workspace: the library keeps D and its tables in
    its own per-device scratch (SEGATTN_NOALLOC_SCRATCH_BYTES), so the C call
    allocates nothing.  dq, dk, dv must be given (this wrapper allocates
    nothing either).  Calls that overlap on one GPU share that scratch and
    race."""
    shape = make_shape(q, k, scale)
    _check_kv(q, k, v)
    _check_stats(q, o, lse)
    _same(do, "do", q.shape, q.dtype)
    _same(dq, "dq", q.shape, dtypes=(torch.bfloat16, torch.float32))
    _same(dk, "dk", k.shape, dq.dtype)
    _same(dv, "dv", k.shape, dq.dtype)
    if accumulate and dq.dtype != torch.float32:
        raise TypeError("accumulate=True needs float32 gradients")
    arr, p, n = _items_arg(items)
    flags = SEGATTN_ACCUMULATE if accumulate else 0
    check(lib().segattn_bwd_noalloc(ctypes.byref(shape), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"),
                                    _DTYPE_CODE[o.dtype], _dev(lse, "lse", torch.float32), _dev(do, "do"), p, n,
                                    _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"), _DTYPE_CODE[dq.dtype], flags,
                                    _stream(stream)))
    return dq, dk, dv


# ------------------------------------------------------------------ offload

def segattn_offload_plan(rows, row_bytes, threshold_bytes):
    """Offload plan of the subsequences (rows[i] rows of row_bytes[i] bytes
    each) for a per-stage transfer volume: returns (alpha, rows_moved, mem,
    peak) as numpy float64 / int64 arrays and a float."""
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    b = np.ascontiguousarray(np.broadcast_to(np.asarray(row_bytes, dtype=np.int64), r.shape))
    n = r.shape[0]
    alpha = np.zeros(n, np.float64)
    moved = np.zeros(n, np.int64)
    mem = np.zeros(n, np.float64)
    peak = ctypes.c_double(0.0)
    f64p = ctypes.POINTER(ctypes.c_double)
    check(lib().segattn_offload_plan(r.ctypes.data_as(_I64P), b.ctypes.data_as(_I64P), n, float(threshold_bytes),
                                     alpha.ctypes.data_as(f64p), moved.ctypes.data_as(_I64P),
                                     mem.ctypes.data_as(f64p), ctypes.byref(peak)))
    return alpha, moved, mem, peak.value


def _rows_view(t, name):
    """(pointer, rows, row bytes, pitch) of a tensor whose dim-0 slices are
    contiguous rows (a slice of a token-major tensor, or a [heads, tokens]
    column block)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dim() == 0:
        raise ValueError(f"{name} must have a row dimension")
    inner = t[0] if t.shape[0] > 0 else t.reshape(-1)
    if t.shape[0] > 0 and not inner.is_contiguous():
        raise ValueError(f"{name}: each row must be contiguous")
    row_bytes = (inner.numel() if t.shape[0] > 0 else 0) * t.element_size()
    pitch = t.stride(0) * t.element_size() if t.shape[0] > 1 else row_bytes
    return ctypes.c_void_p(t.data_ptr()), t.shape[0], row_bytes, pitch


def segattn_copy_rows(dst, src, *, stream=None):
    """Copies the rows of src into dst (same shape; one on the device, the
    other in pinned host memory) asynchronously on `stream` (default: the
    current stream).  The direction follows the devices of src and dst."""
    if dst.shape != src.shape or dst.dtype != src.dtype:
        raise ValueError("dst and src must have the same shape and dtype")
    if src.is_cuda and not dst.is_cuda:
        kind = _lib.SEGATTN_D2H
    elif dst.is_cuda and not src.is_cuda:
        kind = _lib.SEGATTN_H2D
    else:
        raise ValueError("one of dst / src must be a device tensor and the other a host tensor")
    dp, rows, row_bytes, dpitch = _rows_view(dst, "dst")
    sp, _, _, spitch = _rows_view(src, "src")
    dev = src.device if src.is_cuda else dst.device
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    check(lib().segattn_copy_rows(dp, dpitch, sp, spitch, row_bytes, rows, kind, ctypes.c_void_p(s.cuda_stream)))


def segattn_stream_order(event, from_stream, to_stream):
    """Makes to_stream wait for the work enqueued on from_stream so far
    (event: a torch.cuda.Event, recorded on from_stream)."""
    check(lib().segattn_stream_order(ctypes.c_void_p(event.cuda_event), ctypes.c_void_p(from_stream.cuda_stream),
                                     ctypes.c_void_p(to_stream.cuda_stream)))


def segattn_version():
    return lib().segattn_version().decode()
