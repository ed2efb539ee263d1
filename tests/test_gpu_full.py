"""GPU parity at the full sizes of the long-sequence workloads, through the
C ABI, against the float64 oracle on sampled outputs that it can compute one
by one, plus gradient invariants that hold at any size.

  * 131072 tokens, 32 heads, 16 segments, K/V in 16384-token ring blocks
    (Sequence Parallelism blog, Ring Self-Attention: own block first, then
    the earlier ones; InfiniPipe section II-A: partials combined by online
    softmax) -- forward in ring steps merged into an fp32 accumulator,
    backward over the same items in reverse.
  * variable-length batch of 262144 tokens, 32 query / 8 KV heads, sequences
    over 16384 tokens cut into FLOPs-balanced slices (InfiniPipe
    section II-B packed layout; SPPO section 6.1 slice range), typical and
    tail seeds.
  * 1048576 tokens, 40 heads, 64 segments (SPPO section 5.1: one GPU's share
    at million-token scale): forward and backward at full size, sampled rows
    and keys, and full gradients of an independent 8192-token sub-slice.

Sampled outputs: O, LSE and dQ of query rows at every segment / block /
sequence boundary plus seeded random rows; dK and dV of the last keys of a
sequence (a key's gradient needs every later row, so only tail keys are
affordable in float64).  Invariants per (sequence, KV head): sum_j dK_j = 0
(softmax is shift invariant) and sum_j dV_j = sum over the group's query
heads and rows of dO.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import segmented_causal_attention_amd as sa
from gpu_util import Progress, assert_close_g, assert_close_o, ring_steps, say, segments
from synthetic_inputs import WORKLOADS, cu_seqlens, gen_tensors, lognormal_lengths, tail_seed, to_numpy_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _f32(t):
    return to_numpy_f32(t)


def _check_rows(q, k, v, do, o, lse, dq, seq_off, L, h, g, rows, scale, what, grads=True):
    """O, LSE (and dQ) of sequence-local rows `rows` of query head h."""
    sl = slice(seq_off, seq_off + L)
    ks, vs = _f32(k[sl, g]), _f32(v[sl, g])
    ro, rl = oracle.attention_rows(_f32(q[seq_off + rows, h]), ks, vs, rows, scale)
    assert_close_o(o[seq_off + rows, h].float(), ro, f"{what} O h={h}")
    assert_close_o(lse[h, seq_off + rows], rl, f"{what} LSE h={h}")
    if grads:
        rdq = oracle.attention_rows_bwd(_f32(q[seq_off + rows, h]), _f32(do[seq_off + rows, h]), ks, vs, rows, scale)
        assert_close_g(dq[seq_off + rows, h].float(), rdq, f"{what} dQ h={h}")


def _check_tail_keys(q, k, v, do, dk, dv, seq_off, L, g, hq, hkv, nkeys, scale, what):
    """dK, dV of the last nkeys keys of a sequence for KV head g (summed over
    the query heads of its group)."""
    sl = slice(seq_off, seq_off + L)
    keys = np.arange(L - nkeys, L)
    ks, vs = _f32(k[sl, g]), _f32(v[sl, g])
    gk = np.zeros((nkeys, k.shape[2]))
    gv = np.zeros_like(gk)
    for h in range(hq):
        if oracle.kv_head_of(h, hq, hkv) != g:
            continue
        a, b = oracle.attention_keys_bwd(_f32(q[sl, h]), ks, vs, _f32(do[sl, h]), keys, scale)
        gk += a
        gv += b
    assert_close_g(dk[seq_off + keys, g].float(), gk, f"{what} dK g={g}")
    assert_close_g(dv[seq_off + keys, g].float(), gv, f"{what} dV g={g}")


def _check_invariants(do, dk, dv, cu, hq, hkv, what):
    """Per sequence and KV head: sum_j dK_j = 0 and sum_j dV_j = sum dO of the
    group, both relative to the size of the summed terms (float64 sums on
    the device)."""
    T = dk.shape[0]
    cu_t = torch.as_tensor(np.asarray(cu), device=DEV)
    seq = torch.bucketize(torch.arange(T, device=DEV), cu_t[1:], right=True)
    ns = len(cu) - 1
    G = hq // hkv

    def seg_sum(x, absval=False):  # [T, H, d] -> [ns, H, d] in float64, 65536 rows at a time
        out = torch.zeros((ns,) + tuple(x.shape[1:]), dtype=torch.float64, device=DEV)
        for r0 in range(0, T, 65536):
            c = x[r0:r0 + 65536].double()
            out.index_add_(0, seq[r0:r0 + 65536], c.abs() if absval else c)
        return out

    sdk = seg_sum(dk)
    adk = seg_sum(dk, True)
    sdv = seg_sum(dv)
    sdo = seg_sum(do).view(ns, hkv, G, -1).sum(2)
    adv = seg_sum(dv, True)
    rk = float((sdk.abs() / adk.clamp_min(1e-30)).max())
    rv = float(((sdv - sdo).abs() / adv.clamp_min(1e-30)).max())
    say(f"  {what}: max |sum dK| / sum |dK| = {rk:.2e}; max |sum dV - sum dO| / sum |dV| = {rv:.2e}")
    # bf16 outputs carry ~2^-9 relative rounding per entry; the sums of those
    # errors stay far below 1e-2 of the summed magnitudes.
    assert rk < 1e-2 and rv < 1e-2, (rk, rv)


def _whole_heads(q, k, v, do, o, lse, dq, dk, dv, heads, scale, what):
    """Every entry of O, LSE, dQ, dK and dV of whole heads (one causal
    sequence, MHA: KV head = query head) against the float64 oracle run on
    those heads alone -- the unsegmented definition over all rows and keys,
    so the early keys, which gather gradient from every later segment and
    ring block, are compared entry by entry too."""
    hs = list(heads)
    h32 = [_f32(x[:, hs]) for x in (q, k, v, do)]
    ro, rl = oracle.attention_fwd(h32[0], h32[1], h32[2], None, scale, progress=Progress(f"{what} oracle fwd"))
    rq, rk, rv = oracle.attention_bwd(*h32, None, scale, progress=Progress(f"{what} oracle bwd"))
    for i, h in enumerate(hs):
        assert_close_o(o[:, h].float(), ro[:, i], f"{what} whole head {h} O")
        assert_close_o(lse[h], rl[i], f"{what} whole head {h} LSE")
        assert_close_g(dq[:, h].float(), rq[:, i], f"{what} whole head {h} dQ")
        assert_close_g(dk[:, h].float(), rk[:, i], f"{what} whole head {h} dK")
        assert_close_g(dv[:, h].float(), rv[:, i], f"{what} whole head {h} dV")


def _bwd(q, k, v, o, lse, do, items):
    rev = np.ascontiguousarray(np.asarray(items)[::-1])
    return sa.segattn_bwd(q, k, v, o, lse, do, rev)


# ------------------------------------------------------------ ring workload

@pytest.mark.timeout(900)
def test_ring_131072_full_size():
    w = WORKLOADS["ring128k"]
    S, H, d, N, B = w["S"], w["hq"], w["d"], w["N"], w["block"]
    scale = 1 / math.sqrt(d)
    say(f"case ring full seed={w['seed']} S={S} H={H} d={d} N={N} block={B}")
    t = gen_tensors(w["seed"], S, H, H, d, device=DEV)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    b = sa.segattn_partition(S, N)
    items = sa.segattn_ring_items(b, B)
    assert len(items) == 94
    steps = ring_steps(items)
    o = torch.empty((S, H, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((H, S), dtype=torch.float32, device=DEV)
    for s, st in enumerate(steps):
        sa.segattn_fwd(q, k, v, st, o=o, lse=lse, merge_into=s > 0)
    dq, dk, dv = _bwd(q, k, v, o, lse, do, items)
    torch.cuda.synchronize()
    say(f"  {len(steps)} ring steps, {len(items)} items")
    rng = np.random.default_rng(w["seed"])
    blocks = np.arange(B, S, B)
    rows = np.unique(np.concatenate([b[:-1], b[1:] - 1, blocks, blocks - 1, rng.integers(0, S, 16)]))
    for h in (0, H - 1):
        _check_rows(q, k, v, do, o, lse, dq, 0, S, h, h, rows, scale, "ring")
    _check_tail_keys(q, k, v, do, dk, dv, 0, S, 0, H, H, 48, scale, "ring")
    _check_invariants(do, dk, dv, [0, S], H, H, "ring")
    # one whole head through all 8 ring blocks (about 2.5 min of CPU)
    _whole_heads(q, k, v, do, o, lse, dq, dk, dv, [7], scale, "ring")


# ------------------------------------------------------- 32768-token layer

def test_seg_32768_two_whole_heads():
    """The default benchmark workload (32768 tokens, 32 heads, 8 FLOPs-
    balanced segments, bf16 O and gradients, as the benchmark runs it):
    two whole heads compared entry by entry."""
    w = WORKLOADS["seg32k"]
    S, H, d, N = w["S"], w["hq"], w["d"], w["N"]
    scale = 1 / math.sqrt(d)
    say(f"case seg32k whole heads seed={w['seed']} S={S} H={H} d={d} N={N}")
    t = gen_tensors(w["seed"], S, H, H, d, device=DEV)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    items = segments(sa.segattn_partition(S, N))
    o, lse = sa.segattn_fwd(q, k, v, items)
    dq, dk, dv = _bwd(q, k, v, o, lse, do, items)
    torch.cuda.synchronize()
    _whole_heads(q, k, v, do, o, lse, dq, dk, dv, [0, H - 1], scale, "seg32k")


# ------------------------------------------------------ variable-length batch

@pytest.mark.parametrize("which", ["typical", "tail"])
def test_varlen_262144_full_size(which):
    w = WORKLOADS["varlen256k"]
    seed = w["seed"] if which == "typical" else tail_seed(w["seed"])
    hq, hkv, d, cap = w["hq"], w["hkv"], w["d"], w["max_slice"]
    scale = 1 / math.sqrt(d)
    lens = lognormal_lengths(seed, total=w["T"])
    cu = cu_seqlens(lens)
    T = int(cu[-1])
    say(f"case varlen full {which} seed={seed} T={T} sequences={len(lens)} max_len={max(lens)} "
        f"hq={hq} hkv={hkv}")
    t = gen_tensors(seed, T, hq, hkv, d, device=DEV)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    items = sa.segattn_partition_varlen(cu, cap)
    assert [tuple(r) for r in items.tolist()] == oracle.partition_varlen(cu, cap)
    o, lse = sa.segattn_fwd(q, k, v, items, o_dtype=torch.bfloat16)
    dq, dk, dv = _bwd(q, k, v, o, lse, do, items)
    torch.cuda.synchronize()
    say(f"  {len(items)} items")
    rng = np.random.default_rng(seed)
    order = np.argsort(lens)
    picks = {int(order[-1]), int(order[len(order) // 2]), int(order[0])}
    for s in sorted(picks):
        a, L = int(cu[s]), int(lens[s])
        cuts = [int(it[1]) for it in items.tolist() if it[0] == a]
        rows = np.unique(np.clip(np.concatenate([[0, L - 1], cuts, np.asarray(cuts) - 1,
                                                 rng.integers(0, L, 12)]), 0, L - 1))
        what = f"seq{s}(L={L})"
        for h in (0, hq - 1):
            _check_rows(q, k, v, do, o, lse, dq, a, L, h, oracle.kv_head_of(h, hq, hkv), rows, scale, what)
        _check_tail_keys(q, k, v, do, dk, dv, a, L, 0, hq, hkv, min(32, L), scale, what)
    # one short sequence in full: every row and key of its 4 query heads / KV head 0
    s = int(order[len(order) // 4])
    a, L = int(cu[s]), int(lens[s])
    say(f"  full gradients of seq{s} (L={L})")
    sl = slice(a, a + L)
    rq, rk, rv = oracle.attention_bwd(_f32(q[sl, :4]), _f32(k[sl, :1]), _f32(v[sl, :1]), _f32(do[sl, :4]),
                                      None, scale)
    assert_close_g(dq[sl, :4].float(), rq, "short-seq dQ")
    assert_close_g(dk[sl, :1].float(), rk, "short-seq dK")
    assert_close_g(dv[sl, :1].float(), rv, "short-seq dV")
    _check_invariants(do, dk, dv, cu, hq, hkv, "varlen")


def test_varlen_262144_chunked_schedule_full_size():
    """The same 262144-token batch (tail seed: longest sequence 77309) in the
    workload-balanced chunks of InfiniPipe section III-B, Algorithm 1 (K = 4,
    token cap 16384): one forward launch per chunk, then one backward launch
    per chunk in reverse with fp32 gradients accumulating across launches.
    Sampled rows at every chunk boundary of the longest sequence, tail keys
    and the invariants, against the float64 oracle."""
    w = WORKLOADS["varlen256k"]
    seed = tail_seed(w["seed"])
    hq, hkv, d = w["hq"], w["hkv"], w["d"]
    scale = 1 / math.sqrt(d)
    lens = lognormal_lengths(seed, total=w["T"])
    cu = cu_seqlens(lens)
    T = int(cu[-1])
    items, owner, nch, _ = sa.segattn_chunk_varlen(cu, 4, 1.0, 256.0, 16384)
    say(f"case varlen chunked full seed={seed} T={T} max_len={max(lens)} chunks={nch} items={len(items)}")
    t = gen_tensors(seed, T, hq, hkv, d, device=DEV)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    chunks = [items[owner == c] for c in range(nch)]
    o = torch.empty((T, hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((hq, T), dtype=torch.float32, device=DEV)
    for ch in chunks:
        sa.segattn_fwd(q, k, v, ch, o=o, lse=lse)
    dq, dk, dv = (torch.zeros(x.shape, dtype=torch.float32, device=DEV) for x in (q, k, v))
    for ch in reversed(chunks):
        sa.segattn_bwd(q, k, v, o, lse, do, ch[::-1].copy(), dq=dq, dk=dk, dv=dv, accumulate=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed + 7)
    s = int(np.argmax(lens))
    a, L = int(cu[s]), int(lens[s])
    cuts = sorted({int(it[1]) for it in items.tolist() if it[0] == a} | {int(it[2]) for it in items.tolist() if it[0] == a})
    assert len(cuts) >= 4, cuts  # the longest sequence is split by the mesh
    rows = np.unique(np.clip(np.concatenate([[0, L - 1], cuts, np.asarray(cuts) - 1, rng.integers(0, L, 10)]),
                             0, L - 1))
    what = f"chunked seq{s}(L={L})"
    for h in (0, hq - 1):
        _check_rows(q, k, v, do, o, lse, dq, a, L, h, oracle.kv_head_of(h, hq, hkv), rows, scale, what)
    _check_tail_keys(q, k, v, do, dk, dv, a, L, hkv - 1, hq, hkv, 32, scale, what)
    _check_invariants(do, dk, dv, cu, hq, hkv, "chunked varlen")


# ---------------------------------------------------------- 1M-token share

@pytest.fixture(scope="module")
def million():
    w = WORKLOADS["seg1m"]
    say(f"case million inputs seed={w['seed']} S={w['S']} H={w['hq']} d={w['d']}")
    t = gen_tensors(w["seed"], w["S"], w["hq"], w["hkv"], w["d"], device=DEV)
    torch.cuda.synchronize()
    yield w, t
    del t
    torch.cuda.empty_cache()


def test_million_forward_sampled_rows(million):
    w, t = million
    S, H, d, N = w["S"], w["hq"], w["d"], w["N"]
    scale = 1 / math.sqrt(d)
    say(f"case million fwd S={S} H={H} N={N}")
    b = sa.segattn_partition(S, N)
    o, lse = sa.segattn_fwd(t["q"], t["k"], t["v"], segments(b), o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w["seed"])
    # per head: first and last row of every segment plus 128 seeded rows
    rows = np.unique(np.concatenate([b[:-1], b[1:] - 1, rng.integers(0, S, 128)]))
    _check_rows(t["q"], t["k"], t["v"], None, o, lse, None, 0, S, 0, 0, rows, scale, "1M", grads=False)
    rows2 = np.unique(np.concatenate([b[-2:-1], [S - 1], rng.integers(0, S, 30)]))
    _check_rows(t["q"], t["k"], t["v"], None, o, lse, None, 0, S, H - 1, H - 1, rows2, scale, "1M", grads=False)
    # a few rows whose keys span the whole million, against the oracle's
    # softmax over all their keys at once (one key block: no merge on the
    # reference side, so the check does not lean on the merge it tests)
    rows3 = np.array([S // 2, b[-2], S - 1], np.int64)
    h = 7
    ro, rl = oracle.attention_rows(_f32(t["q"][rows3, h]), _f32(t["k"][:, h]), _f32(t["v"][:, h]), rows3, scale,
                                   key_block=S)
    assert_close_o(o[rows3, h].float(), ro, "1M unblocked O")
    assert_close_o(lse[h, rows3], rl, "1M unblocked LSE")


def test_million_backward_sampled(million):
    w, t = million
    S, H, d, N = w["S"], w["hq"], w["d"], w["N"]
    scale = 1 / math.sqrt(d)
    say(f"case million fwd+bwd S={S} H={H} N={N}")
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    items = segments(sa.segattn_partition(S, N))
    o, lse = sa.segattn_fwd(q, k, v, items, o_dtype=torch.bfloat16)
    dq, dk, dv = _bwd(q, k, v, o, lse, do, items)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w["seed"] + 1)
    rows = np.unique(np.concatenate([[0, S - 1], rng.integers(0, S, 14)]))
    h = int(rng.integers(0, H))
    _check_rows(q, k, v, do, o, lse, dq, 0, S, h, h, rows, scale, "1M")
    _check_tail_keys(q, k, v, do, dk, dv, 0, S, h, H, H, 16, scale, "1M")
    del o, lse, dq
    _check_invariants(do, dk, dv, [0, S], H, H, "1M")


def test_million_subslice_full_gradients(million):
    """Rows [t0, t0 + 8192) of the million-token inputs as an independent
    8192-token sequence cut into 32 segments (8 * 32^2 = 8192 keeps the
    segment lengths monotone), full gradients of 4 heads against the oracle."""
    w, t = million
    S, H, d = w["S"], w["hq"], w["d"]
    L, N = 8192, 32
    scale = 1 / math.sqrt(d)
    t0 = int(np.random.default_rng(w["seed"] + 2).integers(0, S - L))
    say(f"case million sub-slice t0={t0} L={L} N={N}")
    sub = {n: t[n][t0:t0 + L].contiguous() for n in ("q", "k", "v", "do")}
    items = segments(sa.segattn_partition(L, N))
    o, lse = sa.segattn_fwd(sub["q"], sub["k"], sub["v"], items, o_dtype=torch.bfloat16)
    dq, dk, dv = _bwd(sub["q"], sub["k"], sub["v"], o, lse, sub["do"], items)
    torch.cuda.synchronize()
    heads = [0, 13, 26, H - 1]
    for h in heads:
        hs = slice(h, h + 1)
        ro, rl = oracle.attention_fwd(_f32(sub["q"][:, hs]), _f32(sub["k"][:, hs]), _f32(sub["v"][:, hs]),
                                      None, scale)
        assert_close_o(o[:, hs].float(), ro, f"sub O h={h}")
        assert_close_o(lse[hs], rl, f"sub LSE h={h}")
        rq, rk, rv = oracle.attention_bwd(_f32(sub["q"][:, hs]), _f32(sub["k"][:, hs]), _f32(sub["v"][:, hs]),
                                          _f32(sub["do"][:, hs]), None, scale)
        assert_close_g(dq[:, hs].float(), rq, f"sub dQ h={h}")
        assert_close_g(dk[:, hs].float(), rk, f"sub dK h={h}")
        assert_close_g(dv[:, hs].float(), rv, f"sub dV h={h}")
