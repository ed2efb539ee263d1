"""GPU parity of the backward path (segattn_bwd_preprocess, segattn_bwd)
against the float64 oracle on identical bf16 inputs.  The GPU forward
supplies O and LSE (as in training); the oracle computes everything from
Q, K, V, dO alone."""

import math

import numpy as np
import pytest
import torch

import oracle
import segmented_causal_attention_amd as sa
from gpu_util import assert_close_g, host64, ring_steps, say, segments
from synthetic_inputs import gen_tensors, to_numpy_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(seed, T, hq, hkv, d, dtype="bf16"):
    t = gen_tensors(seed, T, hq, hkv, d, dtype=dtype, device=DEV)
    return t["q"], t["k"], t["v"], t["do"]


def _h(t):
    return to_numpy_f32(t.to(torch.bfloat16))


def _check(grads, ref, tag=""):
    for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
        assert_close_g(g, r, tag + name)


@pytest.mark.parametrize("T,hq,hkv,d,N,odt,gdt", [
    (1000, 4, 2, 128, 3, torch.bfloat16, torch.bfloat16),
    (1000, 4, 2, 128, 3, torch.float32, torch.float32),
    (777, 2, 1, 64, 2, torch.float32, torch.bfloat16),
    (300, 8, 8, 128, 1, torch.bfloat16, torch.float32),
    (130, 2, 2, 128, 4, torch.float32, torch.float32),
])
def test_segmented_bwd(T, hq, hkv, d, N, odt, gdt):
    say(f"case bwd segmented T={T} hq={hq} hkv={hkv} d={d} N={N} o={odt} g={gdt}")
    q, k, v, do = _inputs(21, T, hq, hkv, d)
    items = segments(sa.segattn_partition(T, N))
    o, lse = sa.segattn_fwd(q, k, v, items, o_dtype=odt)
    grads = sa.segattn_bwd(q, k, v, o, lse, do, items[::-1].copy(), g_dtype=gdt)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(_h(q), _h(k), _h(v), _h(do), None, 1 / math.sqrt(d))
    _check(grads, ref)


def test_fp32_inputs_d64():
    T, d = 1024, 64
    say(f"case bwd fp32-input T={T} d={d}")
    q, k, v, do = _inputs(22, T, 1, 1, d, dtype="fp32")
    items = segments(sa.segattn_partition(T, 4))
    o, lse = sa.segattn_fwd(q, k, v, items, o_dtype=torch.float32)
    grads = sa.segattn_bwd(q, k, v, o, lse, do, items[::-1].copy(), g_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(_h(q), _h(k), _h(v), _h(do), None, 1 / 8)
    _check(grads, ref)


def test_varlen_gqa_bwd():
    lens = [1, 299, 1, 700, 3, 257, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, hq, hkv, d = int(cu[-1]), 8, 2, 128
    say(f"case bwd varlen lens={lens} hq={hq} hkv={hkv}")
    q, k, v, do = _inputs(23, T, hq, hkv, d)
    items = sa.segattn_partition_varlen(cu, 256)
    o, lse = sa.segattn_fwd(q, k, v, items, o_dtype=torch.bfloat16)
    grads = sa.segattn_bwd(q, k, v, o, lse, do, items[::-1].copy())
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(_h(q), _h(k), _h(v), _h(do), cu, 1 / math.sqrt(d))
    _check(grads, ref)


def test_ring_items_bwd():
    S, N, block, hq, d = 1500, 5, 256, 4, 128
    say(f"case bwd ring S={S} N={N} block={block}")
    q, k, v, do = _inputs(24, S, hq, hq, d)
    items = sa.segattn_ring_items(sa.segattn_partition(S, N), block)
    o = torch.zeros((S, hq, d), dtype=torch.float32, device=DEV)
    lse = torch.full((hq, S), -math.inf, dtype=torch.float32, device=DEV)
    for s, step in enumerate(ring_steps(items)):
        sa.segattn_fwd(q, k, v, step, o=o, lse=lse, merge_into=(s > 0))
    grads = sa.segattn_bwd(q, k, v, o, lse, do, items[::-1].copy(), g_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(_h(q), _h(k), _h(v), _h(do), None, 1 / math.sqrt(d))
    _check(grads, ref)


def test_accumulate_one_call_per_segment_in_reverse():
    """SPPO / InfiniPipe order: one backward call per segment, last segment
    first, dK/dV accumulating across calls, equals one call over all."""
    T, hq, hkv, d, N = 1200, 4, 4, 128, 4
    say(f"case bwd accumulate T={T} N={N}")
    q, k, v, do = _inputs(25, T, hq, hkv, d)
    items = segments(sa.segattn_partition(T, N))
    o, lse = sa.segattn_fwd(q, k, v, items, o_dtype=torch.float32)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=DEV)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=DEV)
    for i in reversed(range(N)):
        sa.segattn_bwd(q, k, v, o, lse, do, items[i:i + 1], dq=dq, dk=dk, dv=dv, accumulate=True)
    whole = sa.segattn_bwd(q, k, v, o, lse, do, items[::-1].copy(), g_dtype=torch.float32)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), whole):
        np.testing.assert_allclose(host64(a), host64(b), rtol=2e-5, atol=2e-5)
    ref = oracle.attention_bwd(_h(q), _h(k), _h(v), _h(do), None, 1 / math.sqrt(d))
    _check((dq, dk, dv), ref, "accumulated ")


def test_preprocess_then_d_ready():
    T, hq, d = 600, 2, 128
    say(f"case bwd d_ready T={T}")
    q, k, v, do = _inputs(26, T, hq, hq, d)
    items = segments(sa.segattn_partition(T, 2))
    o, lse = sa.segattn_fwd(q, k, v, items, o_dtype=torch.bfloat16)
    shape = sa.make_shape(q, k)
    ws = torch.empty(sa.segattn_bwd_workspace(shape, items), dtype=torch.uint8, device=DEV)
    sa.segattn_bwd_preprocess(q, k, o, do, items, ws)
    # D rows are plain dot products of the kernel's inputs, stored negated
    delta = ws[: hq * T * 4].view(torch.float32).view(hq, T)
    want = -(o.float() * do.float()).sum(-1).transpose(0, 1)
    np.testing.assert_allclose(host64(delta), host64(want), rtol=1e-4, atol=1e-4)
    g1 = sa.segattn_bwd(q, k, v, o, lse, do, items, workspace=ws, d_ready=True, g_dtype=torch.float32)
    g2 = sa.segattn_bwd(q, k, v, o, lse, do, items, g_dtype=torch.float32)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_preprocess_writes_only_item_rows():
    """D is reduced over the query rows of the items only (a per-segment
    backward call costs its own rows, not the whole batch's)."""
    T, hq, d = 700, 2, 128
    say(f"case bwd D rows T={T}")
    q, k, v, do = _inputs(30, T, hq, hq, d)
    items = np.array([[0, 200, 450, 0, 450]], np.int64)
    o, lse = sa.segattn_fwd(q, k, v, items, o_dtype=torch.bfloat16)
    shape = sa.make_shape(q, k)
    ws = torch.empty(sa.segattn_bwd_workspace(shape, items), dtype=torch.uint8, device=DEV)
    delta = ws[: hq * T * 4].view(torch.float32).view(hq, T)
    delta.fill_(7.0)
    sa.segattn_bwd_preprocess(q, k, o, do, items, ws)
    want = -(o.float() * do.float()).sum(-1).transpose(0, 1)
    torch.cuda.synchronize()
    assert bool((delta[:, :200] == 7.0).all()) and bool((delta[:, 450:] == 7.0).all())
    np.testing.assert_allclose(host64(delta[:, 200:450]), host64(want[:, 200:450]), rtol=1e-4, atol=1e-4)


def test_repeat_run_is_bitwise_identical():
    T, hq, d = 900, 4, 128
    say(f"case bwd determinism T={T}")
    q, k, v, do = _inputs(27, T, hq, 2, d)
    items = segments(sa.segattn_partition(T, 3))
    o, lse = sa.segattn_fwd(q, k, v, items)
    a = sa.segattn_bwd(q, k, v, o, lse, do, items[::-1].copy())
    b = sa.segattn_bwd(q, k, v, o, lse, do, items[::-1].copy())
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_full_size_gradient_invariants():
    """At 32K tokens x 32 heads: per KV head, sum_j dK_j = 0 and
    sum_j dV_j = sum of dO over the rows of the group (exact identities of
    the softmax gradient, so they hold at any size)."""
    S, H, d, N = 32768, 32, 128, 8
    say(f"case bwd invariants S={S} H={H} N={N}")
    q, k, v, do = _inputs(1002, S, H, H, d)
    items = segments(sa.segattn_partition(S, N))
    o, lse = sa.segattn_fwd(q, k, v, items)
    dq, dk, dv = sa.segattn_bwd(q, k, v, o, lse, do, items[::-1].copy(), g_dtype=torch.float32)
    torch.cuda.synchronize()
    sk = dk.double().sum(0)
    scale_k = dk.double().abs().sum(0)
    assert float((sk.abs() / scale_k).max()) < 2e-3
    sv = dv.double().sum(0)
    want = do.double().sum(0)
    rel = float((sv - want).norm() / want.norm())
    say(f"  sum dV rel err {rel:.2e}")
    assert rel < 2e-3
