"""GPU check of the offload entry points on a per-segment schedule (SPPO
sections 5.1-5.2): after each segment's forward, the planned share of its
backward-only rows (Q, O, LSE) is copied to pinned host memory on a second
stream and the device rows are cleared (standing in for releasing them);
before that segment's backward the rows are copied back.  The gradients must
be bit-identical to the same schedule without offloading, and the rows must
really have been cleared before the prefetch."""

import math

import numpy as np
import pytest
import torch

import oracle
import segmented_causal_attention_amd as sa
from gpu_util import say
from synthetic_inputs import gen_tensors, to_numpy_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(q, k, v, do, bounds, offload_rows=None):
    """Per-segment forward, then per-segment backward in reverse (fp32
    gradients accumulated).  offload_rows[i]: rows of segment i to move."""
    T, hq, d = q.shape
    N = len(bounds) - 1
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((hq, T), dtype=torch.float32, device=DEV)
    items = [np.array([[0, bounds[i], bounds[i + 1], 0, bounds[i + 1]]], np.int64) for i in range(N)]
    comp = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    ev = [torch.cuda.Event() for _ in range(N)]
    for e in ev:
        e.record(comp)  # create the events
    host = {}
    cleared_ok = True
    for i in range(N):
        sa.segattn_fwd(q, k, v, items[i], o=o, lse=lse)
        if offload_rows is not None and offload_rows[i] > 0:
            lo, r = bounds[i], offload_rows[i]
            hq_, hl = torch.empty((r, hq, d), dtype=q.dtype, pin_memory=True), torch.empty(
                (r, hq, d), dtype=o.dtype, pin_memory=True)
            hs = torch.empty((hq, r), dtype=torch.float32, pin_memory=True)
            sa.segattn_stream_order(ev[i], comp, copy)  # the copies follow fwd(i)
            sa.segattn_copy_rows(hq_, q[lo:lo + r], stream=copy)
            sa.segattn_copy_rows(hl, o[lo:lo + r], stream=copy)
            sa.segattn_copy_rows(hs, lse[:, lo:lo + r], stream=copy)
            with torch.cuda.stream(copy):  # the rows are free now: clear them
                q[lo:lo + r].zero_()
                o[lo:lo + r].zero_()
                lse[:, lo:lo + r].zero_()
            host[i] = (lo, r, hq_, hl, hs)
    torch.cuda.synchronize()
    for i, (lo, r, *_) in host.items():
        cleared_ok &= bool((q[lo:lo + r] == 0).all()) and bool((o[lo:lo + r] == 0).all())
    dq = torch.zeros(q.shape, dtype=torch.float32, device=DEV)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=DEV)
    # prefetch in reverse on the copy stream; segment i's backward waits for its rows
    ready = {}
    for i in sorted(host, reverse=True):
        lo, r, hq_, hl, hs = host[i]
        sa.segattn_copy_rows(q[lo:lo + r], hq_, stream=copy)
        sa.segattn_copy_rows(o[lo:lo + r], hl, stream=copy)
        sa.segattn_copy_rows(lse[:, lo:lo + r], hs, stream=copy)
        ready[i] = torch.cuda.Event()
        ready[i].record(copy)
    for i in reversed(range(N)):
        if i in ready:
            comp.wait_event(ready[i])
        sa.segattn_bwd(q, k, v, o, lse, do, items[i], dq=dq, dk=dk, dv=dv, accumulate=True)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv, cleared_ok


@pytest.mark.parametrize("T,hq,hkv,N,frac", [(2048, 4, 2, 4, 0.55), (1500, 2, 2, 5, 1.0)])
def test_offload_round_trip_keeps_gradients(T, hq, hkv, N, frac):
    d = 128
    say(f"case offload T={T} hq={hq} hkv={hkv} N={N} frac={frac}")
    t = gen_tensors(31, T, hq, hkv, d, dtype="bf16", device=DEV)
    bounds = [int(x) for x in sa.segattn_partition(T, N)]
    L = [bounds[i + 1] - bounds[i] for i in range(N)]
    row_bytes = hq * d * 2 * 2 + hq * 4
    # threshold: frac of the largest segment's backward-only bytes
    th = frac * max(L) * row_bytes
    alpha, moved, mem, peak = sa.segattn_offload_plan(L, row_bytes, th)
    moved = [int(x) for x in moved]
    moved[-1] = 0  # the last segment's backward comes first: nothing to move
    assert sum(moved) > 0
    base = _run(t["q"].clone(), t["k"], t["v"], t["do"], bounds)
    off = _run(t["q"].clone(), t["k"], t["v"], t["do"], bounds, offload_rows=moved)
    assert off[5], "offloaded device rows were not cleared before the prefetch"
    for a, b, name in zip(base[:5], off[:5], ("O", "LSE", "dQ", "dK", "dV")):
        assert torch.equal(a, b), f"{name} differs after the offload round trip"
    # and the schedule itself computes the attention gradients
    h = [to_numpy_f32(x) for x in (t["q"], t["k"], t["v"], t["do"])]
    rq, rk, rv = oracle.attention_bwd(h[0], h[1], h[2], h[3], None, 1 / math.sqrt(d))
    for got, ref, name in zip(off[2:5], (rq, rk, rv), ("dQ", "dK", "dV")):
        g = got.float().cpu().numpy().astype(np.float64)
        rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
        assert rel <= 1e-2, f"{name} rel-L2 {rel:.3g}"


def test_offload_round_trip_full_size():
    """The 32768-token, 32-head, 8-segment workload (the bench's offload
    case): with the planned share of every segment's Q, O and LSE rows moved
    to pinned host memory and back (33-100 MiB per segment), O, LSE and all
    gradients stay bit-identical to the schedule without offloading."""
    T, hq, hkv, d, N = 32768, 32, 32, 128, 8
    say(f"case offload full size T={T} hq={hq} N={N}")
    t = gen_tensors(32, T, hq, hkv, d, dtype="bf16", device=DEV)
    bounds = [int(x) for x in sa.segattn_partition(T, N)]
    L = [bounds[i + 1] - bounds[i] for i in range(N)]
    row_bytes = hq * d * 2 * 2 + hq * 4
    alpha, moved, mem, peak = sa.segattn_offload_plan(L, row_bytes, 0.55 * max(L) * row_bytes)
    moved = [int(x) for x in moved]
    moved[-1] = 0
    say(f"  rows moved per segment {moved}")
    assert sum(moved) > 0
    base = _run(t["q"].clone(), t["k"], t["v"], t["do"], bounds)
    off = _run(t["q"].clone(), t["k"], t["v"], t["do"], bounds, offload_rows=moved)
    assert off[5], "offloaded device rows were not cleared before the prefetch"
    for a, b, name in zip(base[:5], off[:5], ("O", "LSE", "dQ", "dK", "dV")):
        assert torch.equal(a, b), f"{name} differs after the offload round trip"
