"""Seeded random sweep of the whole path at small sizes, through the C ABI,
against the float64 oracle: head dim 64 / 128, grouped-query ratios 1..8,
FLOPs-balanced segments, variable-length packed batches, ring-order blocks
merged into an fp32 accumulator, bf16 and fp32 inputs and outputs, scales
other than 1/sqrt(d), the accumulate and preprocess-first backward flags,
and key pieces in the forward (SEGATTN_SPLIT_KEYS, drawn from a stream of
its own so that the other draws of a seed do not change).

Each case prints its seed and shape before touching the GPU; the parity bar
is the one of the other GPU tests (O, LSE: max-abs <= 1e-2 and relative-L2
<= 5e-3; dQ, dK, dV: relative-L2 <= 1e-2)."""

import math

import numpy as np
import pytest
import torch

import oracle
import segmented_causal_attention_amd as sa
from gpu_util import assert_close_g, assert_close_o, ring_steps, say, segments
from synthetic_inputs import gen_tensors, to_numpy_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _draw(seed):
    """A valid random configuration (redrawn until the planners accept it)."""
    rng = np.random.default_rng(seed)
    while True:
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 3]))
        hq = hkv * int(rng.choice([1, 2, 3, 4, 6, 8]))
        kind = str(rng.choice(["segments", "varlen", "ring"]))
        cfg = dict(seed=seed, d=d, hq=hq, hkv=hkv, kind=kind,
                   in_dtype="fp32" if rng.random() < 0.2 else "bf16",
                   scale=float(rng.uniform(0.5, 1.5) / math.sqrt(d)),
                   accumulate=bool(rng.random() < 0.3), preprocess=bool(rng.random() < 0.5))
        try:
            if kind == "varlen":
                lens = [int(x) for x in rng.integers(1, 400, int(rng.integers(1, 7)))]
                cu = [0] + list(np.cumsum(lens))
                cap = int(rng.integers(16, 300))
                cfg.update(lens=lens, cu=np.array(cu, np.int64), cap=cap)
                cfg["items"] = np.array(oracle.partition_varlen(cu, cap), np.int64)
                cfg["T"] = int(cu[-1])
            else:
                T = int(rng.integers(1, 900))
                N = int(rng.integers(1, 7))
                b = oracle.partition(T, N)
                cfg.update(T=T, N=N)
                if kind == "ring":
                    blk = int(rng.integers(32, 400))
                    cfg["block"] = blk
                    cfg["items"] = np.array(oracle.ring_items(b, blk), np.int64)
                else:
                    cfg["items"] = segments(np.array(b, np.int64))
        except ValueError:
            continue
        cfg["o_dtype"] = torch.float32 if (kind == "ring" or rng.random() < 0.5) else torch.bfloat16
        cfg["g_dtype"] = torch.float32 if (cfg["accumulate"] or rng.random() < 0.5) else torch.bfloat16
        return cfg


@pytest.mark.parametrize("seed", range(5000, 5048))
def test_random_path(seed):
    c = _draw(seed)
    split = bool(np.random.default_rng([seed, 1]).random() < 0.5)
    T, hq, hkv, d, scale = c["T"], c["hq"], c["hkv"], c["d"], c["scale"]
    say(f"case random seed={seed} kind={c['kind']} T={T} hq={hq} hkv={hkv} d={d} in={c['in_dtype']} "
        f"o={c['o_dtype']} g={c['g_dtype']} acc={c['accumulate']} pre={c['preprocess']} split={split} "
        f"items={len(c['items'])}")
    t = gen_tensors(seed, T, hq, hkv, d, dtype=c["in_dtype"], device=DEV)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    items = c["items"]

    # forward
    if c["kind"] == "ring":
        o = torch.empty((T, hq, d), dtype=torch.float32, device=DEV)
        lse = torch.empty((hq, T), dtype=torch.float32, device=DEV)
        for s, st in enumerate(ring_steps(items)):
            sa.segattn_fwd(q, k, v, st, scale=scale, o=o, lse=lse, merge_into=s > 0, split_keys=split)
    else:
        o, lse = sa.segattn_fwd(q, k, v, items, scale=scale, o_dtype=c["o_dtype"], split_keys=split)

    # backward (items in reverse order)
    rev = np.ascontiguousarray(items[::-1])
    g0 = None
    kw = dict(scale=scale, g_dtype=c["g_dtype"])
    if c["accumulate"]:
        gen = torch.Generator(device=DEV).manual_seed(seed)
        g0 = [torch.randn(x.shape, generator=gen, device=DEV) for x in (q, k, v)]
        kw.update(dq=g0[0].clone(), dk=g0[1].clone(), dv=g0[2].clone(), accumulate=True)
    if c["preprocess"]:
        ws = torch.empty(sa.segattn_bwd_workspace(sa.make_shape(q, k, scale), rev), dtype=torch.uint8, device=DEV)
        sa.segattn_bwd_preprocess(q, k, o, do, rev, ws, scale=scale)
        kw.update(d_ready=True, workspace=ws)
    dq, dk, dv = sa.segattn_bwd(q, k, v, o, lse, do, rev, **kw)
    torch.cuda.synchronize()

    # oracle on the bf16-rounded inputs the kernels stage
    h = [to_numpy_f32(x.to(torch.bfloat16)) for x in (q, k, v, do)]
    cu = c.get("cu")
    ro, rl = oracle.attention_fwd(h[0], h[1], h[2], cu, scale)
    rq, rk, rv = oracle.attention_bwd(h[0], h[1], h[2], h[3], cu, scale)
    if g0 is not None:
        rq, rk, rv = (r + to_numpy_f32(g) for r, g in zip((rq, rk, rv), g0))
    assert_close_o(o.float(), ro, "O")
    assert_close_o(lse, rl, "LSE")
    assert_close_g(dq.float(), rq, "dQ")
    assert_close_g(dk.float(), rk, "dK")
    assert_close_g(dv.float(), rv, "dV")
