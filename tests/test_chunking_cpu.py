"""CPU checks of segattn_chunk_varlen (InfiniPipe section III-B,
Algorithm 1): the library's chunks equal the oracle's exactly -- same float64
operations in the same order -- on random batches and on the log-normal
length mix of the 262144-token varlen workload; argument errors."""

import ctypes

import numpy as np
import pytest

import oracle.chunking as och
import segmented_causal_attention_amd as sa
import synthetic_inputs as synth
from segmented_causal_attention_amd import _lib


def _both(cu, K, a1, a2, cap):
    items, owner, nch, tt = sa.segattn_chunk_varlen(cu, K, a1, a2, cap)
    ritems, rowner = och.chunk_items(cu, K, a1, a2, cap)
    res = och.chunk([b - a for a, b in zip(cu, cu[1:])], K, a1, a2, cap)
    return (items, owner, nch, tt), (ritems, rowner, len(res["chunks"]), res["t_t"])


@pytest.mark.parametrize("seed", range(40))
def test_library_equals_oracle(seed):
    rng = np.random.default_rng(9000 + seed)
    n = int(rng.integers(1, 80))
    lens = np.exp(rng.normal(7.5, 1.6, n)).astype(np.int64) % 70000
    if rng.random() < 0.2:
        lens[rng.integers(0, n)] = 0  # empty sequences are dropped
    if lens.max() == 0:
        lens[0] = 17
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    K = int(rng.integers(1, 7))
    a1 = float(rng.uniform(1e-3, 3.0))
    a2 = float(rng.uniform(0.0, 5000.0)) if rng.random() < 0.7 else 0.0
    cap = int(rng.integers(1, 2 * int(lens.max()) + 2))
    (items, owner, nch, tt), (ritems, rowner, rn, rtt) = _both(cu, K, a1, a2, cap)
    assert [tuple(int(v) for v in r) for r in items] == ritems
    assert owner.tolist() == rowner
    assert nch == rn and tt == rtt


@pytest.mark.parametrize("seed", [1004, 1005, 1006])
def test_varlen_workload_lengths(seed):
    lens = synth.lognormal_lengths(seed, total=262144)
    cu = synth.cu_seqlens(lens)
    for K in (1, 3, 5):
        (items, owner, nch, tt), (ritems, rowner, rn, rtt) = _both(cu, K, 1.0, 2048.0, 16384)
        assert [tuple(int(v) for v in r) for r in items] == ritems
        assert owner.tolist() == rowner and nch == rn and tt == rtt
        # every token row of every sequence in exactly one item
        cover = np.zeros(int(cu[-1]), np.int64)
        for off, lo, hi, klo, khi in items.tolist():
            assert klo == 0 and khi == hi
            cover[off + lo:off + hi] += 1
        assert (cover == 1).all()


def test_capacity_and_errors():
    L = _lib.lib()
    cu = np.array([0, 10, 16, 20, 23, 25], np.int64)
    p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    n, nc, tt = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_double(0)
    items = (_lib.Item * 3)()
    st = L.segattn_chunk_varlen(p, 5, 2, 1.0, 0.0, 8, items, None, 3, ctypes.byref(n), ctypes.byref(nc), None)
    assert st == _lib.SEGATTN_E_CAPACITY and n.value == 6
    bad = [
        (None, 5, 2, 1.0, 0.0, 8),
        (p, 0, 2, 1.0, 0.0, 8),
        (p, 5, 0, 1.0, 0.0, 8),
        (p, 5, 2, 0.0, 0.0, 8),
        (p, 5, 2, 1.0, -1.0, 8),
        (p, 5, 2, float("inf"), 0.0, 8),
        (p, 5, 2, 1.0, float("nan"), 8),
        (p, 5, 2, 1.0, 0.0, 0),
    ]
    for args in bad:
        st = L.segattn_chunk_varlen(*args, None, None, 0, ctypes.byref(n), ctypes.byref(nc), None)
        assert st == _lib.SEGATTN_E_INVALID, args
    dec = np.array([0, 10, 5], np.int64)
    assert L.segattn_chunk_varlen(dec.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 2, 2, 1.0, 0.0, 8, None, None,
                                  0, ctypes.byref(n), ctypes.byref(nc), None) == _lib.SEGATTN_E_INVALID
    empty = np.array([0, 0, 0], np.int64)
    assert L.segattn_chunk_varlen(empty.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 2, 2, 1.0, 0.0, 8, None,
                                  None, 0, ctypes.byref(n), ctypes.byref(nc), None) == _lib.SEGATTN_E_INVALID
    big = np.array([0, 2 ** 31], np.int64)
    assert L.segattn_chunk_varlen(big.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 1, 2, 1.0, 0.0, 8, None,
                                  None, 0, ctypes.byref(n), ctypes.byref(nc), None) == _lib.SEGATTN_E_RANGE
