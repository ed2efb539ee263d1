"""Float64 oracle for causal softmax attention, its log-sum-exp merge and its
gradients, plus the segmented (item-by-item) evaluation.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product library
never calls this module.

Layouts (token-major, packed, as InfiniPipe section II-B's [sum(S), D]):
  q, o, do, dq : [T, Hq, d]      k, v, dk, dv : [T, Hkv, d]
  lse          : [Hq, T]  natural log-sum-exp of the scaled scores of a row
Every input is upcast to float64 before any arithmetic.

What is computed (the pages name the operation -- FlashAttention over the
resident K/V prefix in SPPO section 5.1, "online self-attention" in
InfiniPipe section II-A -- but print no formula; these are the textbook
definitions of softmax attention written out):
  z_ij  = scale * <Q_i, K_j>            for visible j (causal: j <= i)
  LSE_i = log sum_j exp(z_ij)
  P_ij  = exp(z_ij - LSE_i)
  O_i   = sum_j P_ij V_j
and for an upstream gradient dO of f = sum(dO * O):
  D_i   = <dO_i, O_i>
  dV_j  = sum_i P_ij dO_i
  dP_ij = <dO_i, V_j>
  dS_ij = P_ij (dP_ij - D_i)
  dQ_i  = scale * sum_j dS_ij K_j
  dK_j  = scale * sum_i dS_ij Q_i
Grouped-query attention: query head h reads KV head g = floor(h * Hkv / Hq)
(contiguous groups); dK/dV of head g sum over the query heads of its group.

No online softmax and no tiling beyond processing query rows in blocks: every
row's full visible score vector is materialised, max-shifted and
exponentiated with NumPy.
"""

from __future__ import annotations

import numpy as np

_ROW_BLOCK = 256


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """KV head read by query head h: contiguous groups of hq/hkv heads."""
    return (h * hkv) // hq


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _check(q, k, v):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be [T, H, d]")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("shape mismatch")
    if q.shape[1] % k.shape[1]:
        raise ValueError("Hq must be a multiple of Hkv")


def _seq_ranges(T, cu_seqlens):
    if cu_seqlens is None:
        return [(0, T)]
    cu = [int(c) for c in cu_seqlens]
    if cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("bad cu_seqlens")
    return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def _softmax_rows(z):
    """Row-wise softmax of scaled scores with -inf for masked entries.
    Returns (P, LSE); a row with no finite entry gives P = 0, LSE = -inf."""
    m = np.max(z, axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(z - m_safe)
    s = np.sum(e, axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(s))
        p = np.where(empty, 0.0, e / np.where(empty, 1.0, s))
    return p, lse[:, 0]


def attention_fwd(q, k, v, cu_seqlens=None, scale=None, progress=None):
    """Unsegmented causal attention over each packed sequence.
    Returns (O [T,Hq,d] float64, LSE [Hq,T] float64).  progress, if given,
    is called with (rows done, rows in all) after each block of query rows
    (it only reports; nothing it returns is used)."""
    _check(q, k, v)
    T, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    o = np.zeros((T, hq, d))
    lse = np.full((hq, T), -np.inf)
    for (a, b) in _seq_ranges(T, cu_seqlens):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            Q = _f64(q[a:b, h])
            K = _f64(k[a:b, g])
            V = _f64(v[a:b, g])
            for r0 in range(0, b - a, _ROW_BLOCK):
                r1 = min(r0 + _ROW_BLOCK, b - a)
                z = scale * (Q[r0:r1] @ K[:r1].T)
                rows = np.arange(r0, r1)[:, None]
                cols = np.arange(r1)[None, :]
                z = np.where(cols <= rows, z, -np.inf)
                p, l_ = _softmax_rows(z)
                o[a + r0:a + r1, h] = p @ V[:r1]
                lse[h, a + r0:a + r1] = l_
                if progress is not None:
                    progress(h * T + a + r1, hq * T)
    return o, lse


def attention_partial(q, k, v, item, scale=None):
    """Partial attention of one work item: its query rows against the keys
    [k_lo, min(k_hi, q+1)) only.  Returns (O [rows,Hq,d], LSE [Hq,rows]);
    a row with no visible key gives (0, -inf), the merge identity."""
    _check(q, k, v)
    T, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    off, q_lo, q_hi, k_lo, k_hi = (int(x) for x in item)
    rows = q_hi - q_lo
    o = np.zeros((rows, hq, d))
    lse = np.full((hq, rows), -np.inf)
    if rows <= 0 or k_hi <= k_lo:
        return o, lse
    qpos = np.arange(q_lo, q_hi)[:, None]
    kpos = np.arange(k_lo, k_hi)[None, :]
    visible = kpos <= qpos
    for h in range(hq):
        g = kv_head_of(h, hq, hkv)
        Q = _f64(q[off + q_lo:off + q_hi, h])
        K = _f64(k[off + k_lo:off + k_hi, g])
        V = _f64(v[off + k_lo:off + k_hi, g])
        z = np.where(visible, scale * (Q @ K.T), -np.inf)
        p, l_ = _softmax_rows(z)
        o[:, h] = p @ V
        lse[h] = l_
    return o, lse


def merge(o_a, lse_a, o_b, lse_b):
    """Combine two partial results over disjoint key sets A and B.

    Softmax over A u B: O = (e^{l_a} O_a + e^{l_b} O_b) / (e^{l_a} + e^{l_b})
    and LSE = log(e^{l_a} + e^{l_b}); evaluated with the larger LSE m
    factored out (w = e^{l - m}).  If both are -inf (no key in either set)
    the result is the identity (0, -inf).
    o_*: [rows, H, d], lse_*: [H, rows]."""
    o_a, o_b = _f64(o_a), _f64(o_b)
    la, lb = _f64(lse_a), _f64(lse_b)
    m = np.maximum(la, lb)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    wa = np.exp(la - m_safe)
    wb = np.exp(lb - m_safe)
    den = wa + wb
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(den))
        fa = np.where(empty, 0.0, wa / np.where(empty, 1.0, den)).T[:, :, None]
        fb = np.where(empty, 0.0, wb / np.where(empty, 1.0, den)).T[:, :, None]
    return fa * o_a + fb * o_b, lse


def segmented_fwd(q, k, v, items, scale=None):
    """Evaluate item by item, in the order given, merging each partial into
    an accumulator that starts at the identity (0, -inf) for every row.
    Returns (O [T,Hq,d], LSE [Hq,T]); rows no item covers stay (0, -inf)."""
    T, hq, d = q.shape
    o = np.zeros((T, hq, d))
    lse = np.full((hq, T), -np.inf)
    for it in items:
        off, q_lo, q_hi = (int(x) for x in it[:3])
        po, pl = attention_partial(q, k, v, it, scale)
        a, b = off + q_lo, off + q_hi
        o[a:b], lse[:, a:b] = merge(o[a:b], lse[:, a:b], po, pl)
    return o, lse


def attention_bwd(q, k, v, do, cu_seqlens=None, scale=None, progress=None):
    """Gradients of f = sum(dO * O) for unsegmented causal attention over
    each packed sequence.  Returns (dq, dk, dv), float64.  progress as in
    attention_fwd."""
    _check(q, k, v)
    T, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    dq = np.zeros((T, hq, d))
    dk = np.zeros((T, hkv, d))
    dv = np.zeros((T, hkv, d))
    for (a, b) in _seq_ranges(T, cu_seqlens):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            Q = _f64(q[a:b, h])
            K = _f64(k[a:b, g])
            V = _f64(v[a:b, g])
            dO = _f64(do[a:b, h])
            for r0 in range(0, b - a, _ROW_BLOCK):
                r1 = min(r0 + _ROW_BLOCK, b - a)
                z = scale * (Q[r0:r1] @ K[:r1].T)
                rows = np.arange(r0, r1)[:, None]
                cols = np.arange(r1)[None, :]
                z = np.where(cols <= rows, z, -np.inf)
                P, _ = _softmax_rows(z)
                O = P @ V[:r1]
                D = np.sum(dO[r0:r1] * O, axis=1, keepdims=True)
                dv[a:a + r1, g] += P.T @ dO[r0:r1]
                dP = dO[r0:r1] @ V[:r1].T
                dS = P * (dP - D)
                dq[a + r0:a + r1, h] += scale * (dS @ K[:r1])
                dk[a:a + r1, g] += scale * (dS.T @ Q[r0:r1])
                if progress is not None:
                    progress(h * T + a + r1, hq * T)
    return dq, dk, dv


def segmented_bwd(q, k, v, do, items, scale=None):
    """Backward item by item in REVERSE item order (InfiniPipe section II-A:
    a slice's backward runs after those of the slices that follow it;
    section III-A3: dK/dV of earlier slices are completed by the later
    slices' backward).  P is recomputed per item from the final LSE of the
    merged forward, D from the final O.  Returns (dq, dk, dv), float64."""
    _check(q, k, v)
    T, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    o, lse = segmented_fwd(q, k, v, items, scale)
    dq = np.zeros((T, hq, d))
    dk = np.zeros((T, hkv, d))
    dv = np.zeros((T, hkv, d))
    for it in reversed(list(items)):
        off, q_lo, q_hi, k_lo, k_hi = (int(x) for x in it)
        if q_hi <= q_lo or k_hi <= k_lo:
            continue
        qpos = np.arange(q_lo, q_hi)[:, None]
        kpos = np.arange(k_lo, k_hi)[None, :]
        visible = kpos <= qpos
        qa, qb = off + q_lo, off + q_hi
        ka, kb = off + k_lo, off + k_hi
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            Q = _f64(q[qa:qb, h])
            K = _f64(k[ka:kb, g])
            V = _f64(v[ka:kb, g])
            dO = _f64(do[qa:qb, h])
            L = lse[h, qa:qb][:, None]
            with np.errstate(invalid="ignore"):
                P = np.where(visible, np.exp(scale * (Q @ K.T) - L), 0.0)
            D = np.sum(dO * o[qa:qb, h], axis=1, keepdims=True)
            dv[ka:kb, g] += P.T @ dO
            dS = P * (dO @ V.T - D)
            dq[qa:qb, h] += scale * (dS @ K)
            dk[ka:kb, g] += scale * (dS.T @ Q)
    return dq, dk, dv


def attention_rows(q_rows, k_seq, v_seq, row_pos, scale, key_block=65536):
    """O and LSE of selected query rows of ONE head of one sequence: row r
    (sequence position row_pos[r]) attends to keys 0..row_pos[r].
    q_rows [n, d]; k_seq, v_seq [L, d] (that head's K/V of the sequence).
    Keys are processed in blocks and combined with ``merge`` so that a
    million-key row never materialises more than key_block scores.
    Returns (O [n, d], LSE [n])."""
    Q = _f64(q_rows)
    n, d = Q.shape
    pos = np.asarray(row_pos, dtype=np.int64)
    o = np.zeros((n, 1, d))
    lse = np.full((1, n), -np.inf)
    kmax = int(pos.max()) + 1 if n else 0
    for k0 in range(0, kmax, key_block):
        k1 = min(k0 + key_block, kmax)
        K = _f64(k_seq[k0:k1])
        V = _f64(v_seq[k0:k1])
        z = scale * (Q @ K.T)
        z = np.where(np.arange(k0, k1)[None, :] <= pos[:, None], z, -np.inf)
        p, l_ = _softmax_rows(z)
        o, lse = merge(o, lse, (p @ V)[:, None, :], l_[None, :])
    return o[:, 0, :], lse[0]


def attention_rows_bwd(q_rows, do_rows, k_seq, v_seq, row_pos, scale, key_block=65536):
    """dQ of selected query rows of ONE head of one sequence (rows as in
    ``attention_rows``), for the upstream gradient dO of those rows.

    The definition restricted to row i: D_i = <dO_i, O_i> with the row's own
    O_i (from ``attention_rows``), then over the visible keys j <= i
      P_ij = exp(z_ij - LSE_i),  dP_ij = <dO_i, V_j>,
      dS_ij = P_ij (dP_ij - D_i),  dQ_i = scale * sum_j dS_ij K_j,
    accumulated over key blocks.  Returns dQ [n, d]."""
    o, lse = attention_rows(q_rows, k_seq, v_seq, row_pos, scale, key_block)
    Q, dO = _f64(q_rows), _f64(do_rows)
    pos = np.asarray(row_pos, dtype=np.int64)
    D = np.sum(dO * o, axis=1)
    dq = np.zeros_like(Q)
    kmax = int(pos.max()) + 1 if len(pos) else 0
    for k0 in range(0, kmax, key_block):
        k1 = min(k0 + key_block, kmax)
        K = _f64(k_seq[k0:k1])
        V = _f64(v_seq[k0:k1])
        vis = np.arange(k0, k1)[None, :] <= pos[:, None]
        with np.errstate(invalid="ignore"):
            P = np.where(vis, np.exp(scale * (Q @ K.T) - lse[:, None]), 0.0)
        dS = P * (dO @ V.T - D[:, None])
        dq += scale * (dS @ K)
    return dq


def attention_keys_bwd(q_seq, k_seq, v_seq, do_seq, key_pos, scale):
    """dK and dV of selected keys of ONE head of one sequence: key j
    receives from every row i >= j of the sequence.

    The definition restricted to key j: with O_i, LSE_i of the rows
    i >= min(key_pos) (from ``attention_rows``) and D_i = <dO_i, O_i>,
      dV_j = sum_{i >= j} P_ij dO_i,
      dK_j = scale * sum_{i >= j} P_ij (<dO_i, V_j> - D_i) Q_i.
    q_seq, do_seq [L, d] (one query head); k_seq, v_seq [L, d].  For grouped
    heads the caller sums over the query heads of the group.
    Returns (dK [n, d], dV [n, d])."""
    kp = np.asarray(key_pos, dtype=np.int64)
    L = len(q_seq)
    rows = np.arange(int(kp.min()), L)
    o, lse = attention_rows(q_seq[rows], k_seq, v_seq, rows, scale)
    Q, dO = _f64(q_seq[rows]), _f64(do_seq[rows])
    D = np.sum(dO * o, axis=1)
    Kj, Vj = _f64(k_seq[kp]), _f64(v_seq[kp])
    vis = rows[:, None] >= kp[None, :]
    with np.errstate(invalid="ignore"):
        P = np.where(vis, np.exp(scale * (Q @ Kj.T) - lse[:, None]), 0.0)
    dv = P.T @ dO
    dS = P * (dO @ Vj.T - D[:, None])
    dk = scale * (dS.T @ Q)
    return dk, dv
