"""GPU parity of the forward path (segattn_fwd, segattn_merge) against the
float64 oracle on identical bf16 inputs.  Every case prints its name, seed
and shape before touching the GPU."""

import math

import numpy as np
import pytest
import torch

import oracle
import segmented_causal_attention_amd as sa
from gpu_util import assert_close_o, errors, host64, ring_steps, say, segments
from synthetic_inputs import WORKLOADS, gen_tensors, to_numpy_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(seed, T, hq, hkv, d, dtype="bf16"):
    t = gen_tensors(seed, T, hq, hkv, d, dtype=dtype, device=DEV, names=("q", "k", "v"))
    return t["q"], t["k"], t["v"]


def _bf16_host(t):
    """Host float32 copy of t after rounding to bf16 (what the kernels stage)."""
    return to_numpy_f32(t.to(torch.bfloat16))


def test_c1_segmented_fp32_inputs():
    w = WORKLOADS["seg1k_fp32"]
    say(f"case seg1k_fp32 seed={w['seed']} S={w['S']} d={w['d']} N={w['N']} fp32")
    q, k, v = _inputs(w["seed"], w["S"], 1, 1, w["d"], dtype="fp32")
    b = sa.segattn_partition(w["S"], w["N"])
    assert b.tolist() == [0, 512, 724, 887, 1024]
    items = segments(b)
    o, lse = sa.segattn_fwd(q, k, v, items, o_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(_bf16_host(q), _bf16_host(k), _bf16_host(v), scale=1 / 8)
    assert_close_o(o, ro, "O")
    assert_close_o(lse, rl, "LSE")
    # informational: against the oracle on the unrounded fp32 inputs
    fo, fl = oracle.attention_fwd(to_numpy_f32(q), to_numpy_f32(k), to_numpy_f32(v), scale=1 / 8)
    say("  vs fp32-input oracle: O", errors(o, fo), "LSE", errors(lse, fl))


@pytest.mark.parametrize("T,hq,hkv,d,N,odt", [(1000, 4, 2, 128, 3, torch.bfloat16),
                                               (1000, 4, 2, 128, 3, torch.float32),
                                               (777, 2, 1, 64, 2, torch.float32),
                                               (300, 8, 8, 128, 1, torch.bfloat16)])
def test_segmented_bf16(T, hq, hkv, d, N, odt):
    say(f"case segmented T={T} hq={hq} hkv={hkv} d={d} N={N} o={odt}")
    q, k, v = _inputs(11, T, hq, hkv, d)
    items = segments(sa.segattn_partition(T, N))
    o, lse = sa.segattn_fwd(q, k, v, items, o_dtype=odt)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(to_numpy_f32(q), to_numpy_f32(k), to_numpy_f32(v), scale=1 / math.sqrt(d))
    assert_close_o(o, ro, "O")
    assert_close_o(lse, rl, "LSE")


def test_varlen_gqa():
    lens = [1, 299, 1, 700, 3, 257]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, hq, hkv, d = int(cu[-1]), 8, 2, 128
    say(f"case varlen lens={lens} hq={hq} hkv={hkv} d={d}")
    q, k, v = _inputs(12, T, hq, hkv, d)
    items = sa.segattn_partition_varlen(cu, 256)
    assert len(items) > len(lens) - 1
    o, lse = sa.segattn_fwd(q, k, v, items, o_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(to_numpy_f32(q), to_numpy_f32(k), to_numpy_f32(v), cu, 1 / math.sqrt(d))
    assert_close_o(o, ro, "O")
    assert_close_o(lse, rl, "LSE")


@pytest.mark.parametrize("S,N,block", [(1500, 5, 256), (2048, 4, 512)])
def test_ring_order_with_merge_into(S, N, block):
    hq = hkv = 4
    d = 128
    say(f"case ring S={S} N={N} block={block}")
    q, k, v = _inputs(13, S, hq, hkv, d)
    items = sa.segattn_ring_items(sa.segattn_partition(S, N), block)
    o = torch.zeros((S, hq, d), dtype=torch.float32, device=DEV)
    lse = torch.full((hq, S), -math.inf, dtype=torch.float32, device=DEV)
    for s, step in enumerate(ring_steps(items)):
        sa.segattn_fwd(q, k, v, step, o=o, lse=lse, merge_into=(s > 0))
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(to_numpy_f32(q), to_numpy_f32(k), to_numpy_f32(v), scale=1 / math.sqrt(d))
    assert_close_o(o, ro, "O")
    assert_close_o(lse, rl, "LSE")


def test_merge_kernel_in_and_out_of_place():
    rows, h, d = 333, 3, 128
    say(f"case merge rows={rows} h={h} d={d}")
    g = torch.Generator(device="cpu").manual_seed(14)
    oa = torch.randn((rows, h, d), generator=g, dtype=torch.float32)
    ob = torch.randn((rows, h, d), generator=g, dtype=torch.float32)
    la = torch.randn((h, rows), generator=g) * 3
    lb = torch.randn((h, rows), generator=g) * 3
    la[0, :40] = -math.inf
    lb[0, 20:60] = -math.inf
    oa[:40, 0] = 0
    ob[20:60, 0] = 0
    ro, rl = oracle.merge(oa.numpy(), la.numpy(), ob.numpy(), lb.numpy())
    A, LA, Bo, LB = (x.to(DEV) for x in (oa, la, ob, lb))
    o, l = sa.segattn_merge(A, LA, Bo, LB)
    torch.cuda.synchronize()
    assert_close_o(o, ro, "O")
    assert_close_o(l, rl, "LSE")
    assert torch.all(torch.isneginf(l[0, 20:40])).item()
    sa.segattn_merge(A, LA, Bo, LB, o_out=A, lse_out=LA)  # in place into a
    torch.cuda.synchronize()
    assert_close_o(A, ro, "O in place")
    assert_close_o(LA, rl, "LSE in place")
    # a row sub-range of a larger tensor: lse stride = full row count
    A2, LA2 = oa.to(DEV), la.to(DEV)
    r0 = 100
    sa.segattn_merge(A2[r0:], LA2[:, r0:], Bo[r0:], LB[:, r0:], o_out=A2[r0:], lse_out=LA2[:, r0:],
                     rows=rows - r0, lse_stride=rows)
    torch.cuda.synchronize()
    assert_close_o(A2[r0:], ro[r0:], "O sub-range")
    assert np.array_equal(host64(A2[:r0]), oa[:r0].double().numpy())


@pytest.mark.parametrize("rows,h,d", [(1000, 5, 64), (77, 5, 12), (130, 3, 1024)])
def test_merge_kernel_other_head_dims(rows, h, d):
    """The d = 64 fast path and the generic path (any multiple of 4), in and
    out of place, with empty (-inf) rows on either side."""
    say(f"case merge rows={rows} h={h} d={d}")
    g = torch.Generator(device="cpu").manual_seed(rows + d)
    oa = torch.randn((rows, h, d), generator=g, dtype=torch.float32)
    ob = torch.randn((rows, h, d), generator=g, dtype=torch.float32)
    la = torch.randn((h, rows), generator=g) * 3
    lb = torch.randn((h, rows), generator=g) * 3
    la[0, :10] = -math.inf
    lb[0, 5:20] = -math.inf
    oa[:10, 0] = 0
    ob[5:20, 0] = 0
    ro, rl = oracle.merge(oa.numpy(), la.numpy(), ob.numpy(), lb.numpy())
    A, LA, Bo, LB = (x.to(DEV) for x in (oa, la, ob, lb))
    o, l = sa.segattn_merge(A, LA, Bo, LB)
    torch.cuda.synchronize()
    assert_close_o(o, ro, "O")
    assert_close_o(l, rl, "LSE")
    sa.segattn_merge(A, LA, Bo, LB, o_out=Bo, lse_out=LB)  # in place into b
    torch.cuda.synchronize()
    assert_close_o(Bo, ro, "O in place")
    assert_close_o(LB, rl, "LSE in place")


@pytest.mark.parametrize("split", [False, True])
def test_indexing_probe_zero_keys(split):
    """K = 0 makes every visible score exactly 0, so LSE_q = ln(count_q) where
    count_q is the number of keys the item lets row q see; exp(LSE) rounds
    back to that integer, pinning every segment and block boundary (and,
    with key pieces, every piece boundary: the merged LSE is ln of the sum of
    the pieces' counts)."""
    S, N, block = 777, 3, 100
    hq = hkv = 2
    say(f"case probe S={S} N={N} block={block} split={split}")
    q, k, v = _inputs(15, S, hq, hkv, 128)
    k.zero_()
    b = sa.segattn_partition(S, N)
    for it in sa.segattn_ring_items(b, block):
        o, lse = sa.segattn_fwd(q, k, v, it[None, :], o_dtype=torch.float32, split_keys=split)
        torch.cuda.synchronize()
        _, ql, qh, kl, kh = it.tolist()
        rows = np.arange(ql, qh)
        count = np.clip(np.minimum(kh, rows + 1) - kl, 0, None)
        got = host64(lse)[:, ql:qh]
        for hh in range(hq):
            c = np.rint(np.exp(got[hh])).astype(np.int64)
            c[np.isneginf(got[hh])] = 0
            assert np.array_equal(c, count), (it, hh)
        # rows outside the item are untouched
        assert np.all(np.isneginf(host64(lse)[:, :ql])) and np.all(np.isneginf(host64(lse)[:, qh:]))


def test_c2_full_size_sampled_rows():
    w = WORKLOADS["seg32k"]
    S, H, d = w["S"], w["hq"], w["d"]
    say(f"case seg32k full seed={w['seed']} S={S} H={H} d={d} N={w['N']}")
    q, k, v = _inputs(w["seed"], S, H, H, d)
    b = sa.segattn_partition(S, w["N"])
    o, lse = sa.segattn_fwd(q, k, v, segments(b), o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w["seed"])
    rows = np.unique(np.concatenate([b[:-1], b[1:] - 1, rng.integers(0, S, 24)]))
    for h in range(0, H, 5):
        ro, rl = oracle.attention_rows(to_numpy_f32(q[rows, h]), to_numpy_f32(k[:, h]), to_numpy_f32(v[:, h]),
                                       rows, 1 / math.sqrt(d))
        assert_close_o(o[rows, h], ro, f"O h={h}")
        assert_close_o(lse[h, rows], rl, f"LSE h={h}")


@pytest.mark.parametrize("case", ["c1_fp32", "gqa_bf16", "ring_merge", "short_pieces"])
def test_split_keys(case):
    """SEGATTN_SPLIT_KEYS: query tiles of a small launch cut into key pieces
    on separate workgroups, combined by the last piece with the log-sum-exp
    merge.  Against the oracle at the usual bars, close to the unsplit call,
    and bit-identical on a second run."""
    if case == "c1_fp32":
        w = WORKLOADS["seg1k_fp32"]
        T, hq, hkv, d, dt, seed = w["S"], 1, 1, w["d"], "fp32", w["seed"]
        items, odt = segments(sa.segattn_partition(T, w["N"])), torch.float32
    elif case == "gqa_bf16":
        T, hq, hkv, d, dt, seed = 1500, 4, 2, 128, "bf16", 41
        items, odt = segments(sa.segattn_partition(T, 3)), torch.bfloat16
    elif case == "ring_merge":
        T, hq, hkv, d, dt, seed = 1500, 3, 3, 64, "bf16", 42
        items, odt = sa.segattn_ring_items(sa.segattn_partition(T, 5), 256), torch.float32
    else:  # first query tiles see fewer key tiles than the item's piece count: empty pieces
        T, hq, hkv, d, dt, seed = 600, 1, 1, 128, "bf16", 43
        items, odt = np.array([[0, 0, 600, 0, 600]], np.int64), torch.float32
    scale = 1 / math.sqrt(d)
    say(f"case split keys {case} T={T} hq={hq} hkv={hkv} d={d} {dt}")
    q, k, v = _inputs(seed, T, hq, hkv, d, dtype=dt)

    def run(split):
        if case == "ring_merge":
            o = torch.zeros((T, hq, d), dtype=torch.float32, device=DEV)
            lse = torch.full((hq, T), -math.inf, dtype=torch.float32, device=DEV)
            for s_, st in enumerate(ring_steps(items)):
                sa.segattn_fwd(q, k, v, st, o=o, lse=lse, merge_into=s_ > 0, split_keys=split)
            return o, lse
        return sa.segattn_fwd(q, k, v, items, o_dtype=odt, split_keys=split)

    o1, l1 = run(True)
    o2, l2 = run(True)
    o0, l0 = run(False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "split result differs between runs"
    ro, rl = oracle.attention_fwd(_bf16_host(q), _bf16_host(k), _bf16_host(v), None, scale)
    assert_close_o(o1.float(), ro, "O split")
    assert_close_o(l1, rl, "LSE split")
    ma, rel = errors(o1.float(), host64(o0.float()))
    say(f"  split vs unsplit O: max_abs={ma:.2e} rel_l2={rel:.2e}")
    assert rel <= 5e-3


@pytest.mark.parametrize("split,merge", [(False, False), (True, False), (True, True)])
def test_prepared_call_repeats_the_call(split, merge):
    """segattn_fwd_prepare: the prepared callable issues the same C call as
    segattn_fwd (bit-identical outputs), and each call reads the buffers'
    contents at that time (new inputs written into the same tensors give the
    new result)."""
    T, hq, hkv, d = 1100, 2, 1, 64
    say(f"case prepared call split={split} merge={merge} T={T} hq={hq} hkv={hkv} d={d}")
    q, k, v = _inputs(61, T, hq, hkv, d)
    items = segments(sa.segattn_partition(T, 4))
    o = torch.zeros((T, hq, d), dtype=torch.float32, device=DEV)
    lse = torch.full((hq, T), -math.inf, dtype=torch.float32, device=DEV)
    if merge:  # a first partial to merge into, the same for both calls
        sa.segattn_fwd(q, k, v, items, o=o, lse=lse)
    o0, l0 = o.clone(), lse.clone()
    call = sa.segattn_fwd_prepare(q, k, v, items, o=o, lse=lse, merge_into=merge, split_keys=split)
    call()
    ref_o, ref_l = o.clone(), lse.clone()
    o.copy_(o0)
    lse.copy_(l0)
    sa.segattn_fwd(q, k, v, items, o=o, lse=lse, merge_into=merge, split_keys=split)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), "prepared call differs from segattn_fwd"
    # new contents in the same buffers
    q2, k2, v2 = _inputs(62, T, hq, hkv, d)
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    o.copy_(o0)
    lse.copy_(l0)
    call()
    torch.cuda.synchronize()
    if not merge:
        ro, rl = oracle.attention_fwd(_bf16_host(q2), _bf16_host(k2), _bf16_host(v2), None, 1 / math.sqrt(d))
        assert_close_o(o, ro, "O prepared, new inputs")
        assert_close_o(lse, rl, "LSE prepared, new inputs")
    else:
        assert not torch.equal(o, ref_o), "prepared call did not read the new inputs"
