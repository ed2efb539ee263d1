"""Pins of the attention oracle (oracle/attention.py).

Each check reaches the oracle from a direction other than its own code:
PyTorch's float64 scaled_dot_product_attention and autograd (library
routines), pure-Python loops on tiny inputs, closed forms (K = 0, Q = 0,
hard attention), algebraic laws of the merge, central finite differences,
exact gradient invariants, and the identity "segmented + merged ==
unsegmented" that the method rests on (SPPO section 5.1: segment i's queries
attend to the resident K/V of segments 0..i; InfiniPipe section II-A: the
ring runs a multi-step online self-attention).  CPU only.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import planner as PL


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa_ref(q, k, v, scale, causal=True):
    """PyTorch float64 SDPA on [T,H,d] inputs (GQA by repeating K/V heads)."""
    hq, hkv = q.shape[1], k.shape[1]
    rep = hq // hkv
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]
    K = torch.from_numpy(np.repeat(k, rep, axis=1)).permute(1, 0, 2)[None]
    V = torch.from_numpy(np.repeat(v, rep, axis=1)).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def brute_rows(q, k, v, scale):
    """Pure-Python loops, one query row and one key at a time."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    o = np.zeros((T, hq, d))
    lse = np.zeros((hq, T))
    for h in range(hq):
        g = (h * hkv) // hq
        for i in range(T):
            zs = []
            for j in range(i + 1):
                zs.append(scale * sum(float(q[i, h, c]) * float(k[j, g, c]) for c in range(d)))
            m = max(zs)
            s = sum(math.exp(z - m) for z in zs)
            lse[h, i] = m + math.log(s)
            for c in range(d):
                o[i, h, c] = sum(math.exp(zs[j] - lse[h, i]) * float(v[j, g, c]) for j in range(i + 1))
    return o, lse


@pytest.mark.parametrize("T,hq,hkv,d", [(37, 2, 2, 16), (64, 4, 2, 8), (300, 2, 1, 32)])
def test_fwd_matches_torch_sdpa(T, hq, hkv, d):
    q, k, v = rand((T, hq, d), 1), rand((T, hkv, d), 2), rand((T, hkv, d), 3)
    scale = 1 / math.sqrt(d)
    o, lse = A.attention_fwd(q, k, v, scale=scale)
    np.testing.assert_allclose(o, sdpa_ref(q, k, v, scale), rtol=1e-12, atol=1e-12)


def test_fwd_matches_python_loops():
    q, k, v = rand((9, 2, 4), 4), rand((9, 1, 4), 5), rand((9, 1, 4), 6)
    o, lse = A.attention_fwd(q, k, v, scale=0.7)
    ob, lb = brute_rows(q, k, v, 0.7)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("zero", ["k", "q"])
def test_closed_form_uniform_attention(zero):
    """Zero scores: LSE_i = ln(i+1) and O_i = mean of V_0..V_i."""
    T, d = 50, 8
    q, k, v = rand((T, 2, d), 7), rand((T, 2, d), 8), rand((T, 2, d), 9)
    if zero == "k":
        k[:] = 0
    else:
        q[:] = 0
    o, lse = A.attention_fwd(q, k, v, scale=0.3)
    for h in range(2):
        np.testing.assert_allclose(lse[h], np.log(np.arange(1, T + 1)), rtol=0, atol=1e-13)
        np.testing.assert_allclose(o[:, h], np.cumsum(v[:, h], 0) / np.arange(1, T + 1)[:, None],
                                   rtol=1e-12, atol=1e-13)


def test_closed_form_hard_attention():
    """One-hot keys and a large score on key pi(i) <= i: O_i ~ V_pi(i)."""
    T = d = 8
    k = np.eye(T)[:, None, :]
    pi = [i // 2 for i in range(T)]
    q = np.zeros((T, 1, d))
    for i in range(T):
        q[i, 0, pi[i]] = 60.0
    v = rand((T, 1, d), 10)
    o, lse = A.attention_fwd(q, k, v, scale=1.0)
    for i in range(T):
        np.testing.assert_allclose(o[i, 0], v[pi[i], 0], atol=1e-20 + 1e-24 + 1e-12)
        np.testing.assert_allclose(lse[0, i], 60.0 + math.log1p(i * math.exp(-60.0)), atol=1e-12)


def test_varlen_equals_independent_sequences():
    lens = [5, 1, 40, 17]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = cu[-1]
    q, k, v = rand((T, 4, 8), 11), rand((T, 2, 8), 12), rand((T, 2, 8), 13)
    o, lse = A.attention_fwd(q, k, v, cu, scale=0.4)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        os_, ls_ = A.attention_fwd(q[a:b], k[a:b], v[a:b], scale=0.4)
        np.testing.assert_allclose(o[a:b], os_, rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(lse[:, a:b], ls_, rtol=1e-14, atol=1e-14)


def test_gqa_equals_repeated_heads():
    T, hq, hkv, d = 33, 6, 2, 8
    q, k, v = rand((T, hq, d), 14), rand((T, hkv, d), 15), rand((T, hkv, d), 16)
    o, lse = A.attention_fwd(q, k, v, scale=0.5)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    o2, lse2 = A.attention_fwd(q, kr, vr, scale=0.5)
    np.testing.assert_allclose(o, o2, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-14, atol=1e-14)
    assert [A.kv_head_of(h, 32, 8) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]


# ---------------------------------------------------------------- merge laws

def _rand_partial(rows, h, d, seed, empty_frac=0.0):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((rows, h, d))
    l = rng.standard_normal((h, rows)) * 3
    if empty_frac:
        m = rng.random((h, rows)) < empty_frac
        l[m] = -np.inf
        o[m.T] = 0.0
    return o, l


def test_merge_identity_commutative_associative():
    a, b, c = (_rand_partial(20, 3, 5, s, 0.2) for s in (1, 2, 3))
    ident = (np.zeros((20, 3, 5)), np.full((3, 20), -np.inf))
    o, l = A.merge(*a, *ident)
    np.testing.assert_array_equal(l, a[1])
    np.testing.assert_allclose(o, a[0], rtol=0, atol=0)
    ab = A.merge(*a, *b)
    ba = A.merge(*b, *a)
    np.testing.assert_allclose(ab[0], ba[0], rtol=1e-15, atol=1e-15)
    np.testing.assert_array_equal(ab[1], ba[1])
    left = A.merge(*A.merge(*a, *b), *c)
    right = A.merge(*a, *A.merge(*b, *c))
    np.testing.assert_allclose(left[0], right[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(left[1], right[1], rtol=1e-14, atol=1e-14)
    # both empty -> identity, no NaN
    e = A.merge(*ident, *ident)
    assert np.all(e[1] == -np.inf) and np.all(e[0] == 0)


def test_merge_with_itself_adds_ln2():
    a = _rand_partial(10, 2, 4, 5)
    o, l = A.merge(*a, *a)
    np.testing.assert_allclose(o, a[0], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(l, a[1] + math.log(2.0), rtol=1e-15, atol=1e-15)


def test_merge_equals_softmax_over_union():
    """Split the keys of every row into two disjoint sets; merging the two
    partial softmaxes gives the softmax over the union."""
    T, d = 40, 6
    q, k, v = rand((T, 1, d), 20), rand((T, 1, d), 21), rand((T, 1, d), 22)
    o, lse = A.attention_fwd(q, k, v, scale=0.8)
    cut = 17
    pa = A.attention_partial(q, k, v, (0, 0, T, 0, cut), 0.8)
    pb = A.attention_partial(q, k, v, (0, 0, T, cut, T), 0.8)
    om, lm = A.merge(*pa, *pb)
    np.testing.assert_allclose(om, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lm, lse, rtol=1e-14, atol=1e-14)
    # rows below the cut see nothing of block b: partial is the identity
    assert np.all(pb[1][0, :cut] == -np.inf) and np.all(pb[0][:cut] == 0)


# ------------------------------------------------------ segmented identity

@pytest.mark.parametrize("S,N,block", [(257, 1, None), (257, 4, None), (300, 7, None),
                                        (257, 4, 64), (300, 5, 37)])
def test_segmented_equals_unsegmented(S, N, block):
    q, k, v = rand((S, 2, 8), 30), rand((S, 1, 8), 31), rand((S, 1, 8), 32)
    b = PL.partition(S, N)
    if block is None:
        items = [(0, b[i], b[i + 1], 0, b[i + 1]) for i in range(N)]
    else:
        items = PL.ring_items(b, block)
    o, lse = A.attention_fwd(q, k, v, scale=0.35)
    os_, ls_ = A.segmented_fwd(q, k, v, items, 0.35)
    np.testing.assert_allclose(os_, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ls_, lse, rtol=1e-12, atol=1e-13)
    # any arrival order gives the same result
    rev = list(reversed(items))
    os2, ls2 = A.segmented_fwd(q, k, v, rev, 0.35)
    np.testing.assert_allclose(os2, o, rtol=1e-12, atol=1e-13)


def test_segmented_varlen_items():
    cu = [0, 30, 31, 100, 160]
    T = cu[-1]
    q, k, v = rand((T, 4, 8), 33), rand((T, 2, 8), 34), rand((T, 2, 8), 35)
    items = PL.partition_varlen(cu, 25)
    o, lse = A.attention_fwd(q, k, v, cu, 0.3)
    os_, ls_ = A.segmented_fwd(q, k, v, items, 0.3)
    np.testing.assert_allclose(os_, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ls_, lse, rtol=1e-12, atol=1e-13)


def test_attention_rows_matches_full():
    S, d = 700, 16
    q, k, v = rand((S, 1, d), 40), rand((S, 1, d), 41), rand((S, 1, d), 42)
    o, lse = A.attention_fwd(q, k, v, scale=0.25)
    rows = np.array([0, 1, 99, 255, 256, 511, 699])
    orow, lrow = A.attention_rows(q[rows, 0], k[:, 0], v[:, 0], rows, 0.25, key_block=128)
    np.testing.assert_allclose(orow, o[rows, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lrow, lse[0, rows], rtol=1e-13, atol=1e-13)



def test_attention_rows_bwd_matches_full_gradient():
    """dQ of sampled rows, key-blocked, equals the full-gradient oracle's rows
    (which finite differences and autograd pin below)."""
    S, d, scale = 700, 16, 0.25
    q, k, v, do = rand((S, 1, d), 60), rand((S, 1, d), 61), rand((S, 1, d), 62), rand((S, 1, d), 63)
    dq, _, _ = A.attention_bwd(q, k, v, do, None, scale)
    rows = np.array([0, 1, 99, 255, 256, 511, 699])
    got = A.attention_rows_bwd(q[rows, 0], do[rows, 0], k[:, 0], v[:, 0], rows, scale, key_block=128)
    np.testing.assert_allclose(got, dq[rows, 0], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2)])
def test_attention_keys_bwd_matches_full_gradient(hq, hkv):
    """dK/dV of sampled keys (summed over the query heads of each KV head)
    equal the full-gradient oracle's rows."""
    S, d, scale = 300, 8, 0.4
    q, k, v, do = rand((S, hq, d), 64), rand((S, hkv, d), 65), rand((S, hkv, d), 66), rand((S, hq, d), 67)
    _, dk, dv = A.attention_bwd(q, k, v, do, None, scale)
    keys = np.array([0, 7, 150, 298, 299])
    for g in range(hkv):
        gk = np.zeros((len(keys), d))
        gv = np.zeros((len(keys), d))
        for h in range(hq):
            if A.kv_head_of(h, hq, hkv) != g:
                continue
            a, b = A.attention_keys_bwd(q[:, h], k[:, g], v[:, g], do[:, h], keys, scale)
            gk += a
            gv += b
        np.testing.assert_allclose(gk, dk[keys, g], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(gv, dv[keys, g], rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------- backward

def _f(q, k, v, do, cu, scale):
    o, _ = A.attention_fwd(q, k, v, cu, scale)
    return float(np.sum(do * o))


def test_bwd_central_finite_differences():
    """f = sum(dO * O); every input element perturbed by +-h (h = 1e-6)."""
    cu = [0, 4, 9]
    T, hq, hkv, d = 9, 4, 2, 3
    q, k, v, do = rand((T, hq, d), 50), rand((T, hkv, d), 51), rand((T, hkv, d), 52), rand((T, hq, d), 53)
    scale = 0.9
    dq, dk, dv = A.attention_bwd(q, k, v, do, cu, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            fp = _f(q, k, v, do, cu, scale)
            x[idx] = old - h
            fm = _f(q, k, v, do, cu, scale)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 1)])
def test_bwd_matches_torch_autograd(hq, hkv):
    T, d = 70, 16
    q, k, v, do = rand((T, hq, d), 60), rand((T, hkv, d), 61), rand((T, hkv, d), 62), rand((T, hq, d), 63)
    scale = 1 / math.sqrt(d)
    dq, dk, dv = A.attention_bwd(q, k, v, do, None, scale)
    Q = torch.tensor(q, requires_grad=True)
    K = torch.tensor(k, requires_grad=True)
    V = torch.tensor(v, requires_grad=True)
    rep = hq // hkv
    o = torch.nn.functional.scaled_dot_product_attention(
        Q.permute(1, 0, 2)[None], K.repeat_interleave(rep, 1).permute(1, 0, 2)[None],
        V.repeat_interleave(rep, 1).permute(1, 0, 2)[None], is_causal=True, scale=scale)
    (o[0].permute(1, 0, 2) * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, Q.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, K.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, V.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_bwd_exact_invariants():
    """Per sequence and KV head: sum_j dK_j = 0 (softmax is invariant to a
    shift of a row's scores) and sum_j dV_j = sum of dO over the rows and
    the query heads of the group (each P row sums to one)."""
    cu = [0, 50, 51, 130]
    T, hq, hkv, d = 130, 4, 2, 8
    q, k, v, do = rand((T, hq, d), 70), rand((T, hkv, d), 71), rand((T, hkv, d), 72), rand((T, hq, d), 73)
    dq, dk, dv = A.attention_bwd(q, k, v, do, cu, 0.4)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        for g in range(hkv):
            np.testing.assert_allclose(dk[a:b, g].sum(0), 0, atol=1e-12)
            heads = [h for h in range(hq) if A.kv_head_of(h, hq, hkv) == g]
            np.testing.assert_allclose(dv[a:b, g].sum(0), do[a:b, heads].sum((0, 1)), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kind", ["segments", "ring", "varlen"])
def test_segmented_bwd_equals_unsegmented(kind):
    if kind == "varlen":
        cu = [0, 40, 41, 150]
        items = PL.partition_varlen(cu, 30)
    else:
        cu = [0, 200]
        b = PL.partition(200, 5)
        items = ([(0, b[i], b[i + 1], 0, b[i + 1]) for i in range(5)] if kind == "segments"
                 else PL.ring_items(b, 48))
    T = cu[-1]
    q, k, v, do = rand((T, 4, 8), 80), rand((T, 2, 8), 81), rand((T, 2, 8), 82), rand((T, 4, 8), 83)
    ref = A.attention_bwd(q, k, v, do, cu, 0.45)
    got = A.segmented_bwd(q, k, v, do, items, 0.45)
    for r, g in zip(ref, got):
        np.testing.assert_allclose(g, r, rtol=1e-11, atol=1e-12)
