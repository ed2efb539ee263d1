"""Pins of the chunking oracle (InfiniPipe section III-B, Algorithm 1, with
the cost of section III-A2, eq. (1)) to values fixed outside it: the pages'
mesh example, a case worked by hand, the FLOPs-balanced partition (itself
pinned by brute force), brute-force argmins, and exact invariants."""

import math
import os

import numpy as np
import pytest

import oracle.chunking as ch
import oracle.planner as pl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def test_mesh_example_of_the_pages():
    lines = _lines("chunking_mesh_8K4K2K.txt")
    slices = [int(x) for x in lines[0].split()[1:]]
    bounds = [0] + list(np.cumsum(slices))
    for ln in lines[1:]:
        head, *rest = ln.split("|")
        L, *parts = head.split()
        L = int(L)
        split_chunks, tails, shorts = ch.split([L], bounds)
        if parts == ["short"]:
            assert split_chunks == [] and tails == [] and shorts == [(0, L)]
            continue
        assert [s for _, _, s in split_chunks] == [int(x) for x in parts]
        assert [s for _, _, s in tails] == [int(rest[0])]
        # contexts: each piece starts where the previous one ended
        ctx = [c for _, c, _ in split_chunks] + [tails[0][1]]
        assert ctx == list(np.cumsum([0] + [int(x) for x in parts]))


def test_hand_worked_example():
    lines = _lines("chunking_hand_example.txt")
    res = ch.chunk([10, 6, 4, 3, 2], K=2, alpha1=1.0, alpha2=0.0, token_cap=8)
    assert res["mesh"] == [int(x) for x in lines[0].split()[1:]]
    assert res["t_t"] == float(lines[1].split()[1])
    want = []
    for ln in lines[2:]:
        head, slices = ln.split("|")
        kind, ctx = head.split()
        want.append((kind, int(ctx), [tuple(int(v) for v in s.split(":")) for s in slices.split()]))
    got = [(c["kind"], c["context"], c["slices"]) for c in res["chunks"]]
    assert got == want


def test_loosening_terminates_where_the_printed_rule_repeats():
    """In the hand example the bucket with the least time ({6}) cannot take
    the next sequence (T_m), so loosening T_t over all buckets would set the
    same T_t again and again; the reading takes the least over buckets that
    meet T_m and places the sequence."""
    res = ch.chunk([10, 6, 4], K=2, alpha1=1.0, alpha2=0.0, token_cap=8)
    assert res["t_t"] == 67.0
    assert [c["slices"] for c in res["chunks"]] == [[(0, 0, 7)], [(0, 7, 10), (2, 0, 4)], [(1, 0, 6)]]


@pytest.mark.parametrize("L", list(range(1, 200, 7)) + [1024, 16384, 32768, 131072, 1048576])
def test_mesh_with_half_half_is_the_flops_partition(L):
    # f(b) = b^2/2 + b/2 = T(b): the mesh must equal the exact-integer
    # FLOPs-balanced partition of the same length
    for K in range(1, 9):
        if K > L:
            break
        try:
            want = pl.partition(L, K)
        except ValueError:
            continue
        assert ch.mesh(L, K, 0.5, 0.5) == want


@pytest.mark.parametrize("seed", range(40))
def test_mesh_is_the_bruteforce_argmin(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 400))
    K = int(rng.integers(1, min(L, 9) + 1))
    a1 = float(rng.uniform(0.01, 5.0))
    a2 = float(rng.uniform(0.0, 500.0)) if rng.random() < 0.7 else 0.0
    b = ch.mesh(L, K, a1, a2)
    assert b[0] == 0 and b[-1] == L and all(x < y for x, y in zip(b, b[1:]))

    def f(x):
        return a1 * float(x * x) + a2 * float(x)

    for i in range(1, K):
        lo, hi = b[i - 1] + 1, L - (K - i)
        errs = [(abs(float(K) * f(x) - float(i) * f(L)), x) for x in range(lo, hi + 1)]
        assert b[i] == min(errs)[1]


def test_piece_time_closed_form():
    for C, s in ((0, 1), (0, 100), (7, 3), (11705, 2631), (2 ** 20, 2 ** 14)):
        assert ch.piece_time(C, s, 1.0, 0.0) == float((C + s) ** 2 - C ** 2)
        assert ch.piece_time(C, s, 0.5, 0.5) == float(pl.tri(C + s) - pl.tri(C))
        assert ch.piece_time(C, s, 0.0, 3.0) == 3.0 * s


@pytest.mark.parametrize("seed", range(30))
def test_chunks_cover_every_row_once_and_respect_thresholds(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 60))
    lengths = [int(x) for x in np.exp(rng.normal(7.0, 1.5, n)).astype(np.int64) % 40000]
    if max(lengths) == 0:
        lengths[0] = 5
    K = int(rng.integers(1, 6))
    a1, a2 = float(rng.uniform(0.1, 2.0)), float(rng.uniform(0.0, 2000.0))
    cap = int(rng.integers(1, 3 * max(lengths) + 2))
    res = ch.chunk(lengths, K, a1, a2, cap)
    rows = {j: np.zeros(L, np.int64) for j, L in enumerate(lengths)}
    for c in res["chunks"]:
        assert c["slices"]
        for j, lo, hi in c["slices"]:
            assert 0 <= lo < hi <= lengths[j]
            rows[j][lo:hi] += 1
        time = math.fsum(ch.piece_time(lo, hi - lo, a1, a2) for _, lo, hi in c["slices"])
        assert c["time"] == pytest.approx(time, rel=1e-12)
        if c["kind"] == "split":
            assert len(c["slices"]) == 1 and c["context"] == c["slices"][0][1]
            continue
        tokens = sum(hi - lo for _, lo, hi in c["slices"])
        if len(c["slices"]) > 1:
            # joins only ever happen within both thresholds (T_t only grows)
            assert tokens <= cap and c["time"] <= res["t_t"] * (1 + 1e-12)
        if c["kind"] == "hybrid":
            j, lo, _ = c["slices"][0]
            assert c["context"] == lo > 0
            assert all(l2 == 0 for _, l2, _ in c["slices"][1:])
        else:
            assert c["context"] == 0 and all(lo == 0 for _, lo, _ in c["slices"])
    for j, r in rows.items():
        assert (r == 1).all(), f"sequence {j}: rows covered {np.unique(r)}"
    # the mesh pieces of the longest sequence: K - 1 split chunks and a tail
    Lmax = max(lengths)
    jmax = lengths.index(Lmax)
    mine = [c for c in res["chunks"] if c["kind"] == "split" and c["slices"][0][0] == jmax]
    assert len(mine) == len(res["mesh"]) - 2


def test_items_and_errors():
    items, owner = ch.chunk_items([0, 10, 16, 20, 20, 23, 25], 2, 1.0, 0.0, 8)
    # the hand example, packed: sequence offsets 0, 10, 16, (empty), 20, 23
    assert items == [(0, 0, 7, 0, 7), (0, 7, 10, 0, 10), (16, 0, 4, 0, 4), (10, 0, 6, 0, 6),
                     (20, 0, 3, 0, 3), (23, 0, 2, 0, 2)]
    assert owner == [0, 1, 1, 2, 3, 3]
    for bad in (([], 1, 1.0, 0.0, 8), ([0, 5], 1, 0.0, 0.0, 8), ([0, 5], 1, 1.0, -1.0, 8),
                ([0, 5], 1, 1.0, 0.0, 0), ([0, 0], 1, 1.0, 0.0, 8), ([1, 5], 1, 1.0, 0.0, 8)):
        with pytest.raises(ValueError):
            ch.chunk_items(*bad)
