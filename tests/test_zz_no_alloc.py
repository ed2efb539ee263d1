"""segattn_bwd_noalloc -- the backward for callers that cannot allocate --
against segattn_bwd on the same inputs through the C ABI.  Two calls in a
row, the second with a smaller input, so the second runs on scratch that
still holds the first call's D and tables.  The two entry points share their
kernels, plan and D reduction, so the gradients must be bit-identical; they
are also held to the parity bars against the float64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import segmented_causal_attention_amd as sa
from gpu_util import assert_close_g, say, segments
from synthetic_inputs import gen_tensors, to_numpy_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(seed, T, hq, hkv, d, N, gdt, accumulate):
    say(f"case no-alloc bwd seed={seed} T={T} hq={hq} hkv={hkv} d={d} N={N} g={gdt} accumulate={accumulate}")
    t = gen_tensors(seed, T, hq, hkv, d, device=DEV)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    items = segments(sa.segattn_partition(T, N))
    o, lse = sa.segattn_fwd(q, k, v, items)
    rev = items[::-1].copy()
    ref = sa.segattn_bwd(q, k, v, o, lse, do, rev, g_dtype=gdt)
    if accumulate:  # adds onto zeros: 0 + x == x exactly
        out = [torch.zeros_like(x) for x in ref]
    else:  # every entry must be written
        out = [torch.full_like(x, float("nan")) for x in ref]
    sa.segattn_bwd_noalloc(q, k, v, o, lse, do, rev, *out, accumulate=accumulate)
    torch.cuda.synchronize()
    for nm, a, b in zip(("dQ", "dK", "dV"), out, ref):
        assert torch.equal(a, b), f"{nm} differs from segattn_bwd"
    h = [to_numpy_f32(x) for x in (q, k, v, do)]
    rq = oracle.attention_bwd(*h, None, 1 / math.sqrt(d))
    for nm, a, r in zip(("dQ", "dK", "dV"), out, rq):
        assert_close_g(a, r, f"no-alloc {nm}")


def test_noalloc_matches_workspace_entry_two_calls():
    _case(81, 1500, 4, 2, 128, 3, torch.float32, accumulate=True)
    _case(82, 300, 2, 1, 64, 2, torch.bfloat16, accumulate=False)  # smaller, on the first call's scratch
