"""GPU parity on the degenerate shapes of the path: a single token, query
and key tiles with a one-row ragged tail, one-row work items, and packed
batches holding empty and one-token sequences.  Forward and backward
through the C ABI against the float64 oracle on the same bf16 inputs."""

import math

import numpy as np
import pytest
import torch

import oracle
import segmented_causal_attention_amd as sa
from gpu_util import assert_close_g, assert_close_o, host64, say, segments
from synthetic_inputs import gen_tensors, to_numpy_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(seed, T, hq, hkv, d, items, cu=None):
    t = gen_tensors(seed, T, hq, hkv, d, dtype="bf16", device=DEV)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o, lse = sa.segattn_fwd(q, k, v, items, o_dtype=torch.float32)
    grads = sa.segattn_bwd(q, k, v, o, lse, do, items[::-1].copy(), g_dtype=torch.float32)
    torch.cuda.synchronize()
    h = [to_numpy_f32(x) for x in (q, k, v, do)]
    return (q, k, v, do), (o, lse), grads, h


def _check_all(o, lse, grads, h, cu, scale):
    ro, rl = oracle.attention_fwd(h[0], h[1], h[2], cu, scale)
    assert_close_o(o, ro, "O")
    assert_close_o(lse, rl, "LSE")
    for name, g, r in zip(("dQ", "dK", "dV"), grads, oracle.attention_bwd(h[0], h[1], h[2], h[3], cu, scale)):
        assert_close_g(g, r, name)


@pytest.mark.parametrize("d", [128, 64])
def test_single_token(d):
    """One token: the softmax has one term, so O = V, LSE = scale <q, k>,
    dV = dO and dQ = dK = 0 (dS = P (dP - D) with dP = D)."""
    hq, hkv = 2, 1
    say(f"case edge single token d={d}")
    items = segments([0, 1])
    (q, k, v, do), (o, lse), (dq, dk, dv), h = _run(91, 1, hq, hkv, d, items)
    scale = 1 / math.sqrt(d)
    # exact: P = 1 and the normaliser is 1, so O is V itself, and dV is dO
    assert torch.equal(o, v[:, [0, 0]].float()), "O != V"
    # dV = sum over the group's query heads of P dO = dO[h0] + dO[h1] (one fp32 rounding)
    torch.testing.assert_close(dv[:, 0], do[:, 0].float() + do[:, 1].float(), rtol=1e-6, atol=0)
    _, rl = oracle.attention_fwd(h[0], h[1], h[2], None, scale)
    assert np.max(np.abs(host64(lse) - rl)) <= 1e-5
    # dP - D cancels up to fp32 rounding of two different sums
    assert float(dq.abs().max()) <= 1e-4 and float(dk.abs().max()) <= 1e-4


@pytest.mark.parametrize("T,N,hq,hkv,d", [(257, 2, 2, 2, 128), (65, 1, 2, 1, 128), (193, 3, 4, 2, 64)])
def test_one_row_ragged_tail(T, N, hq, hkv, d):
    """T = 64m + 1: the last key tile and the last query tile of the
    sequence hold a single row."""
    say(f"case edge ragged tail T={T} N={N} hq={hq} hkv={hkv} d={d}")
    items = segments(sa.segattn_partition(T, N))
    _, (o, lse), grads, h = _run(92, T, hq, hkv, d, items)
    _check_all(o, lse, grads, h, None, 1 / math.sqrt(d))


def test_one_row_items():
    """Every work item is a single query row (70 items): each workgroup
    has one valid row and every tile is a boundary tile."""
    T, hq, hkv, d = 70, 2, 1, 128
    say(f"case edge one-row items T={T}")
    items = segments(list(range(T + 1)))
    _, (o, lse), grads, h = _run(93, T, hq, hkv, d, items)
    _check_all(o, lse, grads, h, None, 1 / math.sqrt(d))


def test_varlen_with_empty_and_one_token_sequences():
    """Packed batch with empty sequences (repeated offsets) between
    one-token and longer ones, in 64-token slices."""
    lens = [0, 5, 0, 0, 130, 1, 0, 64, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, hq, hkv, d = int(cu[-1]), 4, 2, 128
    say(f"case edge varlen lens={lens}")
    items = sa.segattn_partition_varlen(cu, 64)
    assert all(it[2] > it[1] for it in items.tolist())  # no empty items
    _, (o, lse), grads, h = _run(94, T, hq, hkv, d, items, cu)
    _check_all(o, lse, grads, h, cu, 1 / math.sqrt(d))
