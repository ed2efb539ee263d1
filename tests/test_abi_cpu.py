"""CPU-only checks of the C ABI: the library loads and exports every symbol
include/segattn.h declares, the host planner equals the oracle bit for bit,
and every argument error is reported before anything touches a device."""

import ctypes
import os
import random
import re

import numpy as np
import pytest

from oracle import planner as PL
from segmented_causal_attention_amd import _lib, binding as B
from synthetic_inputs import cu_seqlens, lognormal_lengths, tail_seed

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    txt = open(os.path.join(ROOT, "include", "segattn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(segattn_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_header_symbol():
    L = _lib.lib()
    syms = header_symbols()
    assert len(syms) >= 12
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(_lib.EXPORTS)


def test_status_strings():
    L = _lib.lib()
    for code, name in [(0, "SEGATTN_OK"), (1, "SEGATTN_E_INVALID"), (2, "SEGATTN_E_UNSUPPORTED"),
                       (3, "SEGATTN_E_RANGE"), (4, "SEGATTN_E_CAPACITY"), (5, "SEGATTN_E_WORKSPACE"),
                       (6, "SEGATTN_E_DEVICE")]:
        assert L.segattn_status_string(code).decode() == name


# ------------------------------------------------- planner parity (bit-exact)

@pytest.mark.parametrize("S,N", [(1024, 4), (32768, 8), (131072, 16), (1048576, 64), (8192, 32), (1, 1)])
def test_partition_matches_oracle_configs(S, N):
    assert B.segattn_partition(S, N).tolist() == PL.partition(S, N)


def test_partition_matches_oracle_random():
    rng = random.Random(5)
    for _ in range(20000):
        N = rng.randint(1, 80)
        S = rng.randint(N, max(N, 1 << rng.randint(4, 31))) if rng.random() < 0.9 else rng.randint(N, 3 * N)
        S = min(S, (1 << 31) - 1)
        try:
            want = PL.partition(S, N)
        except ValueError:
            with pytest.raises(B.SegattnError) as e:
                B.segattn_partition(S, N)
            assert e.value.status == _lib.SEGATTN_E_RANGE
            continue
        assert B.segattn_partition(S, N).tolist() == want, (S, N)


def test_varlen_matches_oracle_on_lognormal_batches():
    for seed in [1004, tail_seed(1004), 7, 8, 9]:
        cu = cu_seqlens(lognormal_lengths(seed))
        got = B.segattn_partition_varlen(cu, 16384)
        want = PL.partition_varlen(cu, 16384)
        assert [tuple(r) for r in got.tolist()] == want, seed


def test_varlen_matches_oracle_random_small():
    rng = random.Random(3)
    for _ in range(3000):
        lens = [rng.choice([0, rng.randint(1, 60), rng.randint(1, 400)]) for _ in range(rng.randint(0, 6))]
        cap = rng.randint(1, 80)
        cu = [0] + list(np.cumsum(lens)) if lens else [0]
        try:
            want = PL.partition_varlen(cu, cap)
        except ValueError:
            with pytest.raises(B.SegattnError):
                B.segattn_partition_varlen(cu, cap)
            continue
        got = B.segattn_partition_varlen(cu, cap)
        assert [tuple(r) for r in got.tolist()] == want, (lens, cap)


def test_ring_items_match_oracle():
    rng = random.Random(9)
    for S, N, blk in [(131072, 16, 16384), (1024, 4, 128), (32768, 8, 4096)] + [
            (rng.randint(64, 100000), rng.randint(1, 8), rng.randint(1, 5000)) for _ in range(200)]:
        b = PL.partition(S, N)
        got = B.segattn_ring_items(b, blk)
        assert [tuple(r) for r in got.tolist()] == PL.ring_items(b, blk)


# ------------------------------------------------------------ error paths

def _call_partition(S, N, buf=True):
    L = _lib.lib()
    out = np.zeros(max(N, 0) + 1, dtype=np.int64)
    p = out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)) if buf else None
    return L.segattn_partition(S, N, p), out


def test_partition_errors_write_nothing():
    st, out = _call_partition(10, 0)
    assert st == _lib.SEGATTN_E_INVALID
    st, out = _call_partition(3, 4)
    assert st == _lib.SEGATTN_E_RANGE and not out.any()
    st, out = _call_partition(1 << 31, 4)
    assert st == _lib.SEGATTN_E_RANGE and not out.any()
    st, _ = _call_partition(100, 4, buf=False)
    assert st == _lib.SEGATTN_E_INVALID
    assert "NULL" in _lib.lib().segattn_last_error().decode()


def test_capacity_reports_needed():
    L = _lib.lib()
    cu = np.array([0, 40000, 40010], dtype=np.int64)
    n = ctypes.c_int32(-1)
    items = (_lib.Item * 2)()
    st = L.segattn_partition_varlen(cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 2, 16384, items, 2,
                                    ctypes.byref(n))
    assert st == _lib.SEGATTN_E_CAPACITY and n.value == len(PL.partition_varlen(cu, 16384))
    assert items[0].q_hi == 0  # untouched
    b = np.array([0, 10, 20], dtype=np.int64)
    st = L.segattn_ring_items(b.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 2, 4, items, 1, ctypes.byref(n))
    assert st == _lib.SEGATTN_E_CAPACITY and n.value == 3 + 5


def test_planner_invalid_inputs():
    L = _lib.lib()
    n = ctypes.c_int32(0)
    P64 = ctypes.POINTER(ctypes.c_int64)
    bad_cu = np.array([1, 5], dtype=np.int64)
    assert L.segattn_partition_varlen(bad_cu.ctypes.data_as(P64), 1, 16, None, 0, ctypes.byref(n)) == 1
    dec = np.array([0, 5, 3], dtype=np.int64)
    assert L.segattn_partition_varlen(dec.ctypes.data_as(P64), 2, 16, None, 0, ctypes.byref(n)) == 1
    ok = np.array([0, 5], dtype=np.int64)
    assert L.segattn_partition_varlen(ok.ctypes.data_as(P64), 1, 0, None, 0, ctypes.byref(n)) == 1
    nonmono = np.array([0, 5, 5], dtype=np.int64)
    assert L.segattn_ring_items(nonmono.ctypes.data_as(P64), 2, 4, None, 0, ctypes.byref(n)) == 1
    assert L.segattn_ring_items(ok.ctypes.data_as(P64), 1, 0, None, 0, ctypes.byref(n)) == 1


# Fake, 16-byte aligned "device" addresses: every call below must fail
# validation on the host, so no address is ever dereferenced or launched.
FAKE = ctypes.c_void_p(0x1000)
FAKE2 = ctypes.c_void_p(0x2000)


def _shape(tokens=128, hq=4, hkv=2, d=128, dt=0, scale=0.1):
    return _lib.Shape(tokens, hq, hkv, d, dt, scale)


def _items(rows):
    a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 5))
    return a, a.ctypes.data_as(ctypes.POINTER(_lib.Item)), a.shape[0]


def _fwd(shape, rows, o_dtype=0, flags=0, ws=FAKE, ws_bytes=1 << 20, ptrs=None):
    L = _lib.lib()
    a, p, n = _items(rows)
    q, k, v, o, lse = ptrs or (FAKE, FAKE, FAKE, FAKE, FAKE)
    return L.segattn_fwd(ctypes.byref(shape), q, k, v, p, n, o, o_dtype, lse, flags, ws, ws_bytes, None)


@pytest.mark.parametrize("shape,rows,kw,code", [
    (_shape(d=96), [[0, 0, 8, 0, 8]], {}, _lib.SEGATTN_E_UNSUPPORTED),
    (_shape(hq=3, hkv=2), [[0, 0, 8, 0, 8]], {}, _lib.SEGATTN_E_UNSUPPORTED),
    (_shape(dt=5), [[0, 0, 8, 0, 8]], {}, _lib.SEGATTN_E_INVALID),
    (_shape(scale=float("nan")), [[0, 0, 8, 0, 8]], {}, _lib.SEGATTN_E_INVALID),
    (_shape(scale=0.0), [[0, 0, 8, 0, 8]], {}, _lib.SEGATTN_E_INVALID),
    (_shape(tokens=0), [[0, 0, 8, 0, 8]], {}, _lib.SEGATTN_E_RANGE),
    (_shape(), [[0, 0, 0, 0, 8]], {}, _lib.SEGATTN_E_RANGE),          # empty q range
    (_shape(), [[0, 0, 8, 4, 4]], {}, _lib.SEGATTN_E_RANGE),          # empty k range
    (_shape(), [[0, 0, 8, 0, 9]], {}, _lib.SEGATTN_E_RANGE),          # k_hi > q_hi
    (_shape(), [[100, 0, 29, 0, 8]], {}, _lib.SEGATTN_E_RANGE),       # beyond tokens
    (_shape(), [[-1, 0, 8, 0, 8]], {}, _lib.SEGATTN_E_RANGE),
    (_shape(), [[0, 0, 8, 0, 8], [0, 4, 12, 0, 8]], {}, _lib.SEGATTN_E_INVALID),  # overlapping rows
    (_shape(), [[0, 0, 8, 0, 8]], {"flags": 1, "o_dtype": 0}, _lib.SEGATTN_E_INVALID),  # merge needs fp32
    (_shape(), [[0, 0, 8, 0, 8]], {"flags": 16}, _lib.SEGATTN_E_INVALID),  # unknown flag
    (_shape(), [[0, 0, 8, 0, 8]], {"o_dtype": 7}, _lib.SEGATTN_E_INVALID),
    (_shape(), [[0, 0, 8, 0, 8]], {"ws_bytes": 4}, _lib.SEGATTN_E_WORKSPACE),
    (_shape(), [[0, 0, 8, 0, 8]], {"ws": None}, _lib.SEGATTN_E_WORKSPACE),
    (_shape(), [[0, 0, 8, 0, 8]], {"ptrs": (FAKE, None, FAKE, FAKE, FAKE)}, _lib.SEGATTN_E_INVALID),
    (_shape(), [[0, 0, 8, 0, 8]], {"ptrs": (FAKE, FAKE, ctypes.c_void_p(0x1004), FAKE, FAKE)},
     _lib.SEGATTN_E_INVALID),
])
def test_fwd_argument_errors(shape, rows, kw, code):
    assert _fwd(shape, rows, **kw) == code
    assert _lib.lib().segattn_last_error().decode() != ""


def test_fwd_empty_item_table():
    L = _lib.lib()
    s = _shape()
    assert L.segattn_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, None, 1, FAKE, 0, FAKE, 0, FAKE, 1 << 20, None) == 1
    a, p, _ = _items([[0, 0, 8, 0, 8]])
    assert L.segattn_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, p, 0, FAKE, 0, FAKE, 0, FAKE, 1 << 20, None) == 1


def test_workspace_queries():
    s = _shape(tokens=1000, hq=8, hkv=2)
    a, p, n = _items([[0, 0, 500, 0, 500], [0, 500, 1000, 0, 1000]])
    nb = ctypes.c_size_t(0)
    L = _lib.lib()
    assert L.segattn_fwd_workspace(ctypes.byref(s), p, n, ctypes.byref(nb)) == 0 and nb.value >= 2 * 32
    assert L.segattn_bwd_workspace(ctypes.byref(s), p, n, ctypes.byref(nb)) == 0
    assert nb.value >= 8 * 1000 * 4  # D = <dO, O> rows live in the workspace


def test_bwd_argument_errors():
    L = _lib.lib()
    s = _shape()

    def bwd(rows, g_dtype=0, flags=0, ws_bytes=1 << 20, o_dtype=0):
        a, p, n = _items(rows)
        return L.segattn_bwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, o_dtype, FAKE, FAKE, p, n, FAKE, FAKE, FAKE,
                             g_dtype, flags, FAKE2, ws_bytes, None)

    assert bwd([[0, 0, 8, 0, 8]], g_dtype=0, flags=2) == _lib.SEGATTN_E_INVALID   # accumulate needs fp32
    assert bwd([[0, 0, 8, 0, 8]], flags=16) == _lib.SEGATTN_E_INVALID
    assert bwd([[0, 0, 8, 0, 8]], ws_bytes=8) == _lib.SEGATTN_E_WORKSPACE
    assert bwd([[0, 0, 8, 0, 8]], g_dtype=3) == _lib.SEGATTN_E_INVALID
    # identical query ranges must be adjacent items
    assert bwd([[0, 0, 8, 0, 4], [0, 8, 16, 0, 16], [0, 0, 8, 4, 8]]) == _lib.SEGATTN_E_INVALID
    # partially overlapping query ranges
    assert bwd([[0, 0, 8, 0, 8], [0, 4, 16, 0, 16]]) == _lib.SEGATTN_E_INVALID


def test_merge_argument_errors():
    L = _lib.lib()
    assert L.segattn_merge(0, 1, 128, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.segattn_merge(8, 1, 126, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.segattn_merge(8, 1, 128, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.segattn_merge(8, 1, 1028, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.SEGATTN_E_UNSUPPORTED
    assert L.segattn_merge(8, 1, 128, 8, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.segattn_merge(8, 1, 128, 8, FAKE, ctypes.c_void_p(0x1001), FAKE, FAKE, FAKE, FAKE, None) == 1


def test_bwd_noalloc_argument_errors():
    """The no-allocation backward rejects SEGATTN_D_READY and any call whose
    scratch need exceeds its fixed array, before touching a device."""
    L = _lib.lib()
    a, p, n = _items([[0, 0, 8, 0, 8]])
    s = _shape()

    def call(shape, items, flags=0, g_dtype=1):
        a_, p_, n_ = _items(items)
        return L.segattn_bwd_noalloc(ctypes.byref(shape), FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, p_, n_, FAKE, FAKE,
                                     FAKE, g_dtype, flags, None)

    assert call(s, [[0, 0, 8, 0, 8]], flags=_lib.SEGATTN_D_READY) == _lib.SEGATTN_E_INVALID
    assert call(s, [[0, 0, 8, 0, 8]], flags=_lib.SEGATTN_ACCUMULATE, g_dtype=0) == _lib.SEGATTN_E_INVALID
    assert call(s, [[0, 0, 8, 0, 4], [0, 8, 16, 0, 16], [0, 0, 8, 4, 8]]) == _lib.SEGATTN_E_INVALID
    # D alone: 4 * hq * tokens bytes; 8 heads x 2^22 tokens = 128 MiB > 64 MiB
    big = _shape(tokens=1 << 22, hq=8, hkv=8)
    assert call(big, [[0, 0, 1 << 22, 0, 1 << 22]]) == _lib.SEGATTN_E_WORKSPACE
    msg = L.segattn_last_error().decode()
    assert "no-allocation" in msg and str(_lib.SEGATTN_NOALLOC_SCRATCH_BYTES) in msg, msg
    # the workspace the same call would need from segattn_bwd is what does not fit
    nb = ctypes.c_size_t(0)
    a2, p2, n2 = _items([[0, 0, 1 << 22, 0, 1 << 22]])
    assert L.segattn_bwd_workspace(ctypes.byref(big), p2, n2, ctypes.byref(nb)) == 0
    assert nb.value > _lib.SEGATTN_NOALLOC_SCRATCH_BYTES


def test_varlen_capacity_query_fails_like_the_call():
    """A slice cap so small that the balanced partition of a sequence would
    hold an empty slice is E_RANGE for the capacity query as well, not a
    count that the writing call then refuses."""
    L = _lib.lib()
    cu = np.array([0, 62210], np.int64)
    n = ctypes.c_int32(0)
    st = L.segattn_partition_varlen(cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 1, 2, None, 0,
                                    ctypes.byref(n))
    assert st == _lib.SEGATTN_E_RANGE, (st, n.value)
