"""Planted mistakes in the oracle (CPU only): each plausible slip must be
caught by one of the pins, which shows the pins have teeth."""

import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import planner as PL

from test_oracle_attention import rand, sdpa_ref
from test_oracle_partition import read_golden


def test_dropped_linear_term_in_causal_work_is_caught(monkeypatch):
    g = read_golden("partition_S1024_N4.txt")
    monkeypatch.setattr(PL, "tri", lambda x: int(x) * int(x) // 2)
    assert PL.partition(1024, 4) != g["bounds"] or PL.segment_work(g["bounds"]) != g["work"]


def test_interleaved_gqa_mapping_is_caught(monkeypatch):
    T, hq, hkv, d = 20, 4, 2, 8
    q, k, v = rand((T, hq, d), 1), rand((T, hkv, d), 2), rand((T, hkv, d), 3)
    monkeypatch.setattr(A, "kv_head_of", lambda h, a, b: h % b)
    o, _ = A.attention_fwd(q, k, v, scale=0.3)
    assert not np.allclose(o, sdpa_ref(q, k, v, 0.3), rtol=1e-6, atol=1e-6)


def test_wrong_merge_weights_are_caught():
    def bad_merge(o_a, lse_a, o_b, lse_b):  # swaps the two weights
        return A.merge(o_a, lse_b, o_b, lse_a)

    T, d = 30, 4
    q, k, v = rand((T, 1, d), 4), rand((T, 1, d), 5), rand((T, 1, d), 6)
    o, lse = A.attention_fwd(q, k, v, scale=0.7)
    pa = A.attention_partial(q, k, v, (0, 0, T, 0, 11), 0.7)
    pb = A.attention_partial(q, k, v, (0, 0, T, 11, T), 0.7)
    om, _ = bad_merge(*pa, *pb)
    assert not np.allclose(om, o, rtol=1e-6, atol=1e-6)


def test_off_by_one_causal_mask_is_caught():
    """Strict mask (k < q) instead of k <= q: the K = 0 closed form
    LSE_i = ln(i+1) fails."""
    T, d = 12, 4
    q, k, v = rand((T, 1, d), 7), np.zeros((T, 1, d)), rand((T, 1, d), 8)
    o, lse = A.attention_partial(q, k, v, (0, 1, T, 0, T), 1.0)  # rows 1.. see keys <= q
    # a strict mask would give ln(i) for row i; the oracle must give ln(i+1)
    assert np.allclose(lse[0], np.log(np.arange(2, T + 1)))
    assert not np.allclose(lse[0], np.log(np.arange(1, T)))


@pytest.mark.parametrize("mut", ["sign_D", "no_scale_dk"])
def test_gradient_slips_are_caught_by_finite_differences(mut):
    T, hq, hkv, d = 6, 2, 1, 3
    q, k, v, do = rand((T, hq, d), 9), rand((T, hkv, d), 10), rand((T, hkv, d), 11), rand((T, hq, d), 12)
    scale = 0.8
    dq, dk, dv = A.attention_bwd(q, k, v, do, None, scale)
    if mut == "sign_D":
        # dS = P (dP + D): recompute dq for head 0 the wrong way
        o, lse = A.attention_fwd(q, k, v, scale=scale)
        z = scale * q[:, 0] @ k[:, 0].T
        z = np.where(np.tril(np.ones((T, T))) > 0, z, -np.inf)
        P = np.exp(z - lse[0][:, None])
        D = np.sum(do[:, 0] * o[:, 0], 1, keepdims=True)
        bad = scale * (P * (do[:, 0] @ v[:, 0].T + D)) @ k[:, 0]
        target, mine = dq[:, 0], bad
    else:
        target, mine = dk, dk / scale
    h = 1e-6

    def f():
        o, _ = A.attention_fwd(q, k, v, scale=scale)
        return float(np.sum(do * o))

    x = q if mut == "sign_D" else k
    num = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        old = x[idx]
        x[idx] = old + h
        fp = f()
        x[idx] = old - h
        fm = f()
        x[idx] = old
        num[idx] = (fp - fm) / (2 * h)
    num = num[:, 0] if mut == "sign_D" else num
    assert np.allclose(target, num, rtol=1e-6, atol=1e-8)
    assert not np.allclose(mine, num, rtol=1e-3, atol=1e-5)
    assert math.isfinite(float(np.sum(mine)))


# ----------------------------------------------------------------- chunking
# Planted slips in the chunking oracle (InfiniPipe section III-B, Algorithm
# 1); the pages' example, the hand-worked case and the partition equality
# must catch each.

from oracle import chunking as CH  # noqa: E402

from test_oracle_chunking import _lines  # noqa: E402


def _hand_chunks():
    res = CH.chunk([10, 6, 4, 3, 2], K=2, alpha1=1.0, alpha2=0.0, token_cap=8)
    return [(c["kind"], c["context"], c["slices"]) for c in res["chunks"]], res["t_t"]


def _hand_want():
    lines = _lines("chunking_hand_example.txt")
    want = []
    for ln in lines[2:]:
        head, slices = ln.split("|")
        kind, ctx = head.split()
        want.append((kind, int(ctx), [tuple(int(v) for v in x.split(":")) for x in slices.split()]))
    return want, float(lines[1].split()[1])


def test_chunking_pins_hold_unmutated():
    assert _hand_chunks() == _hand_want()


def test_buckets_tried_by_descending_metric_is_caught(monkeypatch):
    monkeypatch.setattr(CH, "bucket_order",
                        lambda bs: sorted(bs, key=lambda b: (-(b["time"] / float(b["tokens"])), b["id"])))
    assert _hand_chunks() != _hand_want()


def test_shorts_by_increasing_time_is_caught(monkeypatch):
    monkeypatch.setattr(CH, "short_order", lambda shorts, a1, a2: sorted(shorts, key=lambda js: (js[1], js[0])))
    assert _hand_chunks() != _hand_want()


def test_time_threshold_of_the_whole_sequence_is_caught(monkeypatch):
    monkeypatch.setattr(CH, "initial_time_threshold", lambda L, K, a1, a2: a1 * float(L * L) + a2 * float(L))
    assert _hand_chunks() != _hand_want()


def test_dropped_linear_cost_term_is_caught(monkeypatch):
    real = CH.mesh
    monkeypatch.setattr(CH, "mesh", lambda L, K, a1, a2: real(L, K, a1, 0.0))
    # with alpha1 = alpha2 = 1/2 the mesh must be the FLOPs partition
    assert any(CH.mesh(L, K, 0.5, 0.5) != PL.partition(L, K) for L in (37, 100, 1000) for K in (2, 3, 5))
    monkeypatch.setattr(CH, "mesh", real)
    real_piece = CH.piece_time
    monkeypatch.setattr(CH, "piece_time", lambda c, s, a1, a2: real_piece(c, s, a1, 0.0))
    assert CH.piece_time(7, 3, 0.5, 0.5) != float(PL.tri(10) - PL.tri(7))


def test_mesh_cut_at_boundaries_not_inside_is_caught(monkeypatch):
    """Cutting a sequence at boundaries <= L (instead of < L) turns an exact
    12288-token sequence into 8K + 4K split chunks with an empty tail."""
    def bad_split(lengths, bounds):
        inner = bounds[1:-1]
        sc, tails, shorts = [], [], []
        for j, L in enumerate(lengths):
            cuts = [b for b in inner if b <= L]
            if not cuts:
                shorts.append((j, L))
                continue
            starts = [0] + cuts
            for a, b in zip(starts[:-1], cuts):
                sc.append((j, a, b - a))
            tails.append((j, cuts[-1], L - cuts[-1]))
        return sc, tails, shorts

    lines = _lines("chunking_mesh_8K4K2K.txt")
    bounds = [0] + list(np.cumsum([int(x) for x in lines[0].split()[1:]]))
    pinned = {}
    for ln in lines[1:]:
        head, *rest = ln.split("|")
        L, *parts = head.split()
        pinned[int(L)] = None if parts == ["short"] else ([int(x) for x in parts], int(rest[0]))
    monkeypatch.setattr(CH, "split", bad_split)
    caught = False
    for L, want in pinned.items():
        sc, tails, shorts = CH.split([L], bounds)
        got = None if shorts else ([s for _, _, s in sc], tails[0][2])
        caught |= got != want
    assert caught
