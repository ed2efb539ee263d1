"""GPU parity where the online softmax works hardest: scores that rise along
the sequence, so that every row's running maximum grows by more than 8
(base 2) on every 64-key tile and the lazy rescale runs on each of them,
and a large score scale that makes P nearly one-hot.  Forward and backward
against the float64 oracle on the same bf16 inputs, every output at the
usual bars.

The rising ramp also gives every key a large shared component (up to
1.5 T along one axis).  dQ_i = scale sum_j dS_ij K_j with sum_j dS_ij = 0, so
dQ only depends on how K varies near the row; the kernel measures keys from
the query row's own key, which keeps the bf16 rounding of dS and the
forward's bf16 P (through D) from carrying the shared component into dQ.
These cases hold dQ to the same relative-L2 bar as every other gradient."""

import math

import numpy as np
import pytest
import torch

import oracle
import segmented_causal_attention_amd as sa
from gpu_util import G_REL_L2, O_MAX_ABS, O_REL_L2, errors, say, segments
from synthetic_inputs import gen_tensors, to_numpy_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check(q, k, v, do, items, scale, cu=None):
    o, lse = sa.segattn_fwd(q, k, v, items, scale=scale, o_dtype=torch.float32)
    grads = sa.segattn_bwd(q, k, v, o, lse, do, items[::-1].copy(), scale=scale, g_dtype=torch.float32)
    torch.cuda.synchronize()
    h = [to_numpy_f32(x) for x in (q, k, v, do)]
    ro, rl = oracle.attention_fwd(h[0], h[1], h[2], cu, scale)
    rq, rk, rv = oracle.attention_bwd(h[0], h[1], h[2], h[3], cu, scale)
    errs = {"O": errors(o, ro), "LSE": errors(lse, rl)}
    for g, r, nm in zip(grads, (rq, rk, rv), ("dQ", "dK", "dV")):
        errs[nm] = errors(g, r)
    for nm, (ma, rl2) in errs.items():
        say(f"  {nm}: max_abs={ma:.3e} rel_l2={rl2:.3e}")
    for nm in ("O", "LSE"):
        assert errs[nm][0] <= O_MAX_ABS and errs[nm][1] <= O_REL_L2, (nm, errs[nm])
    for nm in ("dQ", "dK", "dV"):
        assert errs[nm][1] <= G_REL_L2, (nm, errs[nm])


@pytest.mark.parametrize("T,N,hq,hkv,d", [(1000, 2, 2, 1, 128), (700, 3, 2, 2, 64)])
def test_running_maximum_grows_on_every_tile(T, N, hq, hkv, d):
    scale = 1 / math.sqrt(d)
    # score of key j for every row ~ scale * 1.5 j: per 64-key tile the row
    # maximum grows by 64 * 1.5 * scale * log2(e) > 8 in base 2 (d <= 128)
    step = 1.5 if d == 128 else 1.1
    say(f"case sharp rising scores T={T} N={N} hq={hq} hkv={hkv} d={d} step={step}")
    t = gen_tensors(71, T, hq, hkv, d, dtype="bf16", device=DEV)
    u = torch.zeros(d, device=DEV)
    u[0] = 1.0
    q = (u + 0.1 * t["q"].float()).to(torch.bfloat16)
    ramp = (step * torch.arange(T, device=DEV, dtype=torch.float32)).view(T, 1, 1)
    k = (ramp * u + 0.5 * t["k"].float()).to(torch.bfloat16)
    assert 64 * step * scale * math.log2(math.e) > 8
    items = segments(sa.segattn_partition(T, N))
    _check(q, k, t["v"], t["do"], items, scale)


def test_large_scale_nearly_one_hot():
    T, N, hq, hkv, d = 900, 3, 4, 2, 128
    scale = 6 / math.sqrt(d)
    say(f"case sharp large scale T={T} N={N} scale={scale:.3f}")
    t = gen_tensors(72, T, hq, hkv, d, dtype="bf16", device=DEV)
    items = segments(sa.segattn_partition(T, N))
    _check(t["q"], t["k"], t["v"], t["do"], items, scale)


def test_sharp_varlen_slices():
    """Rising scores in every sequence of a varlen batch cut into
    FLOPs-balanced slices."""
    lens = [333, 600, 91]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, hq, hkv, d = int(cu[-1]), 2, 1, 128
    scale = 1 / math.sqrt(d)
    say(f"case sharp varlen lens={lens}")
    t = gen_tensors(73, T, hq, hkv, d, dtype="bf16", device=DEV)
    u = torch.zeros(d, device=DEV)
    u[0] = 1.0
    local = torch.cat([torch.arange(L, device=DEV, dtype=torch.float32) for L in lens]).view(T, 1, 1)
    q = (u + 0.1 * t["q"].float()).to(torch.bfloat16)
    k = (1.5 * local * u + 0.5 * t["k"].float()).to(torch.bfloat16)
    items = sa.segattn_partition_varlen(cu, 256)
    _check(q, k, t["v"], t["do"], items, scale, cu)


@pytest.mark.parametrize("T,hq,hkv,d,ring,odt,off", [
    (800, 4, 2, 128, False, torch.bfloat16, 16.0),
    (900, 6, 3, 64, True, torch.float32, 8.0),
])
def test_keys_share_a_large_offset(T, hq, hkv, d, ring, odt, off):
    """Every key shifted by the same vector (off in every coordinate): the
    softmax of each row is unchanged (the shift adds a per-row constant to
    its scores), so dQ is unchanged in exact arithmetic, but the keys now
    share a component of norm off sqrt(d).  GQA, segments or ring blocks
    with merges, bf16 or fp32 forward output."""
    scale = 1 / math.sqrt(d)
    say(f"case shared key offset T={T} hq={hq} hkv={hkv} d={d} ring={ring} o={odt} off={off}")
    t = gen_tensors(74, T, hq, hkv, d, dtype="bf16", device=DEV)
    k = (t["k"].float() + off).to(torch.bfloat16)
    bounds = sa.segattn_partition(T, 3)
    if ring:
        from gpu_util import ring_steps
        items = sa.segattn_ring_items(bounds, 256)
        o = torch.zeros((T, hq, d), dtype=torch.float32, device=DEV)
        lse = torch.full((hq, T), -math.inf, dtype=torch.float32, device=DEV)
        for s, step in enumerate(ring_steps(items)):
            sa.segattn_fwd(t["q"], k, t["v"], step, scale=scale, o=o, lse=lse, merge_into=(s > 0))
    else:
        items = segments(bounds)
        o, lse = sa.segattn_fwd(t["q"], k, t["v"], items, scale=scale, o_dtype=odt)
    grads = sa.segattn_bwd(t["q"], k, t["v"], o, lse, t["do"], items[::-1].copy(), scale=scale,
                           g_dtype=torch.float32)
    torch.cuda.synchronize()
    h = [to_numpy_f32(x) for x in (t["q"], k, t["v"], t["do"])]
    ref = oracle.attention_bwd(h[0], h[1], h[2], h[3], None, scale)
    for g, r, nm in zip(grads, ref, ("dQ", "dK", "dV")):
        ma, rl2 = errors(g, r)
        say(f"  {nm}: max_abs={ma:.3e} rel_l2={rl2:.3e}")
        assert rl2 <= G_REL_L2, (nm, ma, rl2)
