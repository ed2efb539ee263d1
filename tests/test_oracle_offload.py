"""Pins of the offload-plan oracle (SPPO section 5.2, sequence-aware
offloading) to values fixed outside the oracle: the reading guide's worked
example, hand-worked cases, and the closed form of the memory recurrence."""

import math
import os

import numpy as np
import pytest

import oracle.offload as off

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_fixture(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = [float(x) for x in rest]
    return vals


def test_worked_example():
    g = read_fixture("offload_A50_70_T40.txt")
    alpha, mem, peak = off.plan_offload(g["act_gb"], g["threshold_gb"][0])
    assert alpha == pytest.approx(g["alpha"], rel=1e-15)
    assert round(alpha[1], 2) == g["alpha1_rounded"][0]
    assert (1 - alpha[0]) * g["act_gb"][0] == pytest.approx(g["kept_after_stage0_gb"][0], rel=1e-12)
    assert mem == pytest.approx(g["mem_gb"], rel=1e-15)
    assert mem[1] + g["resident_kv_gb"][0] == pytest.approx(g["gpu_use_at_stage1_with_kv_gb"][0], rel=1e-15)
    assert peak == pytest.approx(80.0, rel=1e-15)


def test_small_subsequence_moves_whole_and_recurrence_uses_previous_stage():
    # Worked by hand: A = 30, 70 and a 40 threshold.  alpha0 = 1 (30 < 40, all
    # of it moves), alpha1 = 40/70.  M1 = 30 + 70 - 1*30 = 70: the volume moved
    # during stage 1 is stage 0's (30), not stage 1's own (40), which would
    # give 60.
    alpha, mem, peak = off.plan_offload([30, 70], 40)
    assert alpha == [1.0, 40 / 70]
    assert mem == [30.0, 70.0]
    assert peak == 70.0


def test_zero_volume_and_errors():
    alpha, mem, _ = off.plan_offload([0, 10], 5)
    assert alpha == [0.0, 0.5] and mem == [0.0, 10.0]
    for bad in (([], 1), ([1, 2], 0), ([1, -1], 1)):
        with pytest.raises(ValueError):
            off.plan_offload(*bad)


@pytest.mark.parametrize("seed", range(20))
def test_closed_form_and_invariants(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    act = [float(x) for x in rng.uniform(0.1, 100.0, n)]
    th = float(rng.uniform(1.0, 80.0))
    alpha, mem, peak = off.plan_offload(act, th)
    for a, x in zip(alpha, act):
        assert 0.0 <= a <= 1.0
        # alpha_i A_i = threshold wherever the subsequence is large enough
        assert a * x == pytest.approx(min(th, x), rel=1e-12)
    # M_i = sum_{j<=i} A_j - sum_{j<i} alpha_j A_j
    for i in range(n):
        want = math.fsum(act[: i + 1]) - math.fsum(alpha[j] * act[j] for j in range(i))
        assert mem[i] == pytest.approx(want, rel=1e-12, abs=1e-9)
    assert peak == max(mem)


def test_ratios_fall_as_subsequences_grow():
    # SPPO section 5.2: for subsequences ordered s0 <= s1 <= ... the ratios
    # come out alpha0 >= alpha1 >= ...
    act = [10.0, 20.0, 35.0, 60.0, 90.0]
    alpha, _, _ = off.plan_offload(act, 25.0)
    assert all(a >= b for a, b in zip(alpha, alpha[1:]))


def test_offload_rows():
    assert off.offload_rows(0.8, 100) == 80
    assert off.offload_rows(40 / 70, 7000) == 4000
    assert off.offload_rows(1.0, 37) == 37
    assert off.offload_rows(0.0, 37) == 0
    # never more bytes than the threshold when alpha < 1
    for rows, row_bytes, th in ((1000, 48, 10000.0), (4096, 16384, 3e7), (9, 1, 4.0)):
        a = min(1.0, th / (rows * row_bytes))
        r = off.offload_rows(a, rows)
        assert r * row_bytes <= th + 1e-9 and r <= rows
