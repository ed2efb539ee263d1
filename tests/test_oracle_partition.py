"""Pins of the planner oracle (oracle/planner.py) against brute force,
closed forms, a hand-worked example and exact coverage invariants.
CPU only."""

import math
import os
import random

import pytest

from oracle import planner as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_partition(S, N):
    """Independent path: scan every b in [0, S] for every boundary."""
    tot = S * (S + 1) // 2
    b = [0]
    for i in range(1, N):
        b.append(min(range(S + 1),
                     key=lambda x: (abs(N * (x * (x + 1) // 2) - i * tot), x)))
    b.append(S)
    return b


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = [int(x) for x in rest]
    return vals


def test_hand_worked_example():
    g = read_golden("partition_S1024_N4.txt")
    S, N = g["S"][0], g["N"][0]
    assert P.partition(S, N) == g["bounds"]
    assert P.segment_work(g["bounds"]) == g["work"]


def test_bruteforce_all_small():
    for S in range(1, 161):
        for N in range(1, min(S, 12) + 1):
            ref = brute_partition(S, N)
            if all(ref[i] < ref[i + 1] for i in range(N)):
                assert P.partition(S, N) == ref, (S, N)
            else:
                with pytest.raises(ValueError):
                    P.partition(S, N)


def test_bruteforce_random_medium():
    rng = random.Random(7)
    for _ in range(120):
        S = rng.randint(200, 4096)
        N = rng.randint(1, 16)
        ref = brute_partition(S, N)
        assert P.partition(S, N) == ref, (S, N)


def _real_root(i, N, S):
    # x(x+1)/2 = i*T(S)/N  ->  x = (-1 + sqrt(1 + 8 i T(S) / N)) / 2
    return (-1.0 + math.sqrt(1.0 + 8.0 * i * (S * (S + 1) / 2.0) / N)) / 2.0


@pytest.mark.parametrize("S,N", [(1024, 4), (32768, 8), (131072, 16), (1048576, 64),
                                 (8192, 32), (65536, 16), (100000, 7)])
def test_invariants_and_closed_form(S, N):
    b = P.partition(S, N)
    assert b[0] == 0 and b[-1] == S and len(b) == N + 1
    assert all(b[i] < b[i + 1] for i in range(N))
    # each boundary lies within one token of the real root of the balance
    # equation (the quadratic causal-work term of InfiniPipe eq. (1))
    for i in range(1, N):
        assert abs(b[i] - _real_root(i, N, S)) <= 1.0
    # continuous limit b_i ~ S*sqrt(i/N)
    for i in range(1, N):
        assert abs(b[i] - S * math.sqrt(i / N)) <= 1.5
    # work per segment within S + 2 pairs of the ideal T(S)/N
    ideal = (S * (S + 1) // 2) / N
    for w in P.segment_work(b):
        assert abs(w - ideal) <= S + 2
    assert sum(P.segment_work(b)) == S * (S + 1) // 2
    # "start with longer subsequences": lengths non-increasing when S >= 8 N^2
    if S >= 8 * N * N:
        lens = [b[i + 1] - b[i] for i in range(N)]
        assert all(lens[i] >= lens[i + 1] for i in range(N - 1)), lens


def test_monotone_lengths_random():
    rng = random.Random(11)
    for _ in range(300):
        N = rng.randint(1, 48)
        S = rng.randint(8 * N * N, 8 * N * N + 200000)
        b = P.partition(S, N)
        lens = [b[i + 1] - b[i] for i in range(N)]
        assert all(lens[i] >= lens[i + 1] for i in range(N - 1)), (S, N, lens)


def test_partition_errors():
    with pytest.raises(ValueError):
        P.partition(3, 4)
    with pytest.raises(ValueError):
        P.partition(10, 0)
    # N = 1 is the whole sequence
    assert P.partition(5, 1) == [0, 5]


def _visible_pairs_brute(items, T):
    """Set of (token_q, token_k) pairs covered, asserting no duplicates."""
    seen = set()
    for (off, ql, qh, kl, kh) in items:
        for q in range(ql, qh):
            for k in range(kl, min(kh, q + 1)):
                pair = (off + q, off + k)
                assert pair not in seen, pair
                seen.add(pair)
    return seen


def test_varlen_items_cover_every_pair_once():
    cu = [0, 5, 5, 40, 41, 130, 200]
    items = P.partition_varlen(cu, max_slice=30)
    got = _visible_pairs_brute(items, cu[-1])
    want = set()
    for s in range(len(cu) - 1):
        for q in range(cu[s + 1] - cu[s]):
            for k in range(q + 1):
                want.add((cu[s] + q, cu[s] + k))
    assert got == want


@pytest.mark.parametrize("L", [1, 16384, 16385, 20000, 32768, 65536, 100000, 131072])
def test_varlen_slicing_rule(L):
    cap = 16384
    items = P.partition_varlen([0, L], cap)
    if L <= cap:
        assert items == [(0, 0, L, 0, L)]
        return
    n = len(items)
    assert n >= 2
    b = [it[1] for it in items] + [items[-1][2]]
    assert b == P.partition(L, n)
    assert all(it[3] == 0 and it[4] == it[2] for it in items)
    assert b[1] <= cap
    # minimality: with one slice fewer the first slice would exceed the cap
    if n > 2:
        assert P.partition(L, n - 1)[1] > cap
    # first (longest) slice of a FLOPs-balanced cut is ~ L / sqrt(n)
    assert abs(b[1] - L / math.sqrt(n)) <= 1.5


def test_ring_items_cover_every_pair_once():
    for S, N, B in [(100, 4, 16), (257, 5, 64), (64, 1, 64), (90, 3, 7)]:
        b = P.partition(S, N)
        items = P.ring_items(b, B)
        got = _visible_pairs_brute(items, S)
        assert len(got) == S * (S + 1) // 2
        # own (diagonal) block first, then strictly descending blocks
        for st in P.ring_steps(items)[0]:
            assert st[4] == st[2]
        for i in range(N):
            seg = [it for it in items if it[1] == b[i]]
            assert [it[3] for it in seg] == sorted((it[3] for it in seg), reverse=True)
            assert seg[-1][3] == 0


def test_ring_items_large_config_counts():
    b = P.partition(131072, 16)
    items = P.ring_items(b, 16384)
    per_seg = {}
    pairs = 0
    for (off, ql, qh, kl, kh) in items:
        per_seg[(ql, qh)] = per_seg.get((ql, qh), 0) + 1
        # visible pairs of the item: rows q in [ql,qh) with keys [kl, min(kh, q+1))
        lo = max(ql, kl)
        # rows below kl see nothing; rows q >= kh see all kh-kl keys
        for_rows_full = max(0, qh - max(ql, kh)) * (kh - kl)
        diag_hi = min(qh, kh)
        diag = sum(q + 1 - kl for q in range(lo, diag_hi)) if diag_hi > lo else 0
        pairs += for_rows_full + diag
        assert kh - kl <= 16384
    assert pairs == 131072 * 131073 // 2
    counts = [per_seg[(b[i], b[i + 1])] for i in range(16)]
    assert counts == [-(-b[i + 1] // 16384) for i in range(16)]
    steps = P.ring_steps(items)
    assert len(steps) == 8 and steps[0][0][3] == 16384  # segment 0 owns block 1 first
