"""GPU parity of the chunked varlen schedule (InfiniPipe section III-B,
Algorithm 1): the items of segattn_chunk_varlen, run one forward launch per
chunk in chunk order and one backward launch per chunk in reverse order
(fp32 gradients accumulating across launches, as the split chunks of a
sequence complete the earlier slices' dK/dV), against the float64 oracle of
unsegmented causal attention on the same bf16 inputs; and a single launch
over all chunk items, which must equal the per-chunk schedule's forward."""

import math

import numpy as np
import pytest
import torch

import oracle
import segmented_causal_attention_amd as sa
from gpu_util import assert_close_g, assert_close_o, host64, say
from synthetic_inputs import gen_tensors, to_numpy_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("lens,K,cap,hq,hkv,d", [
    ([700, 300, 2, 129, 64, 511, 1], 3, 600, 4, 2, 128),
    ([1200, 1200, 90, 45, 33], 2, 500, 2, 1, 64),
    ([1500], 4, 2000, 2, 2, 128),
])
def test_chunked_schedule_matches_oracle(lens, K, cap, hq, hkv, d):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    items, owner, nch, tt = sa.segattn_chunk_varlen(cu, K, 1.0, 256.0, cap)
    say(f"case chunking lens={lens} K={K} cap={cap} hq={hq} hkv={hkv} d={d} chunks={nch} items={len(items)}")
    t = gen_tensors(61, T, hq, hkv, d, dtype="bf16", device=DEV)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    chunks = [items[owner == c] for c in range(nch)]
    o = torch.empty((T, hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((hq, T), dtype=torch.float32, device=DEV)
    for ch in chunks:
        sa.segattn_fwd(q, k, v, ch, o=o, lse=lse)
    grads = [torch.zeros(x.shape, dtype=torch.float32, device=DEV) for x in (q, k, v)]
    for ch in reversed(chunks):
        sa.segattn_bwd(q, k, v, o, lse, do, ch[::-1].copy(), dq=grads[0], dk=grads[1], dv=grads[2],
                       accumulate=True)
    o1, lse1 = sa.segattn_fwd(q, k, v, items, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    h = [to_numpy_f32(x) for x in (q, k, v, do)]
    ro, rl = oracle.attention_fwd(h[0], h[1], h[2], cu, 1 / math.sqrt(d))
    rq, rk, rv = oracle.attention_bwd(h[0], h[1], h[2], h[3], cu, 1 / math.sqrt(d))
    assert_close_o(o.float(), ro, "O")
    assert_close_o(lse, rl, "LSE")
    for g, r, nm in zip(grads, (rq, rk, rv), ("dQ", "dK", "dV")):
        assert_close_g(g, r, nm)
    # one launch over every chunk's items computes the same rows
    assert np.array_equal(host64(o1), host64(o)) and np.array_equal(host64(lse1), host64(lse))
