"""CPU checks of the offload entry points: the library's plan equals the
oracle's exactly (same float64 operations in the same order), and the copy /
ordering calls reject bad arguments before touching the device."""

import ctypes

import numpy as np
import pytest

import oracle
import segmented_causal_attention_amd as sa
from segmented_causal_attention_amd import _lib


def _oracle_plan(rows, row_bytes, th):
    act = [int(r) * int(b) for r, b in zip(rows, row_bytes)]
    alpha, mem, peak = oracle.plan_offload(act, th)
    moved = [oracle.offload_rows(a, r) for a, r in zip(alpha, rows)]
    return alpha, moved, mem, peak


def test_worked_example_through_the_library():
    alpha, moved, mem, peak = sa.segattn_offload_plan([50, 70], 1, 40)
    assert alpha.tolist() == [0.8, 40 / 70]
    assert moved.tolist() == [40, 40]
    assert mem.tolist() == [50.0, 80.0] and peak == 80.0


@pytest.mark.parametrize("seed", range(30))
def test_plan_matches_oracle_exactly(seed):
    rng = np.random.default_rng(7000 + seed)
    n = int(rng.integers(1, 70))
    rows = rng.integers(0, 200000, n)
    row_bytes = rng.integers(1, 20000, n) if rng.random() < 0.5 else np.full(n, int(rng.integers(1, 20000)))
    th = float(rng.uniform(1.0, 2e9))
    alpha, moved, mem, peak = sa.segattn_offload_plan(rows, row_bytes, th)
    ra, rm, rmem, rpeak = _oracle_plan(rows.tolist(), row_bytes.tolist(), th)
    assert alpha.tolist() == ra
    assert moved.tolist() == rm
    assert mem.tolist() == rmem
    assert peak == rpeak


def test_plan_errors():
    for args in (([], [], 1.0), ([1, 2], [1, 1], 0.0), ([1, -2], [1, 1], 1.0), ([1], [1], float("inf")),
                 ([2 ** 62], [4], 1.0)):
        with pytest.raises(_lib.SegattnError) as e:
            sa.segattn_offload_plan(*args)
        assert e.value.status == _lib.SEGATTN_E_INVALID


def test_copy_and_order_argument_errors_without_device_work():
    L = _lib.lib()
    vp = ctypes.c_void_p
    buf = ctypes.create_string_buffer(64)
    p = ctypes.cast(buf, vp)
    # bad kind, negative sizes, NULL pointers, short pitch: rejected on the host
    assert L.segattn_copy_rows(p, 64, p, 64, 16, 2, 7, None) == _lib.SEGATTN_E_INVALID
    assert L.segattn_copy_rows(p, 64, p, 64, -1, 2, _lib.SEGATTN_D2H, None) == _lib.SEGATTN_E_INVALID
    assert L.segattn_copy_rows(None, 64, p, 64, 16, 2, _lib.SEGATTN_D2H, None) == _lib.SEGATTN_E_INVALID
    assert L.segattn_copy_rows(p, 8, p, 64, 16, 2, _lib.SEGATTN_H2D, None) == _lib.SEGATTN_E_INVALID
    # an empty copy is a no-op (no HIP call)
    assert L.segattn_copy_rows(None, 0, None, 0, 16, 0, _lib.SEGATTN_D2H, None) == _lib.SEGATTN_OK
    assert L.segattn_stream_order(None, None, None) == _lib.SEGATTN_E_INVALID
