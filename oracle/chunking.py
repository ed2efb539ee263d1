"""Oracle for workload-balanced sequence chunking of a variable-length batch
(InfiniPipe, section III-B "Sequence Processor", Algorithm 1, with the
computation cost of section III-A2, eq. (1)).

TEST INFRASTRUCTURE ONLY (see the package docstring): the product library
never calls this module.

What the pages fix, and the readings taken where they are silent:

* Cost.  Eq. (1) charges a slice s with context C the time
  alpha1((C + s)^2 - C^2) + alpha2 s, and a chunk the sum over its slices.
  The factor 1/N and the per-chunk constant beta1/d_p are common to every
  chunk on one device and are left out.  (C + s)^2 - C^2 = s(2C + s) is
  formed exactly in integers, then scaled in float64.
* Mesh.  The longest sequence L is cut into K slices of equal
  time: boundary b_i is the integer minimising |K f(b) - i f(L)| with
  f(b) = alpha1 b^2 + alpha2 b (ties to the smaller b), found from the
  positive root of K f(b) = i f(L) and a check of its integer neighbours.
  With alpha1 = alpha2 = 1/2, f(b) = b(b+1)/2 and the mesh is the
  FLOPs-balanced segment partition.
* Split.  A sequence is cut at every inner mesh boundary that lies
  strictly inside it; the pieces before the last cut are split chunks (one
  slice each, its context the tokens before it), the last piece is its tail
  slice.  A sequence no mesh boundary falls inside is a short sequence.
  This gives the pages' example: with a mesh {8K, 4K, 2K} a sequence longer
  than 12K becomes an 8K and a 4K split chunk and a remainder.
* Thresholds.  T_t starts at one mesh slice's time f(L)/K.  The pages omit
  how T_m follows from the token capacity; here T_m is the caller's token
  capacity per bucket.  A bucket's token count is the sum of its slices
  (a tail's context is not in it: those keys and values belong to the
  split chunks).
* Buckets.  One bucket per tail slice, kept ordered by
  tot_time / tot_tokens ascending (ties: the older bucket first); short
  sequences taken longest-time first (ties: earlier sequence first).  A
  short sequence opens a new bucket when even the bucket with the fewest
  tokens would exceed T_m; otherwise it joins the first bucket in metric
  order within both thresholds.  When none qualifies, T_t is loosened to
  the least bucket time plus the sequence's time and the placement is
  retried.  Reading: the least is taken over the buckets that meet T_m --
  over all buckets, as printed, the retry can repeat forever when the
  bucket with the least time is the one over T_m.
* Output.  Split chunks (by sequence, then position), then
  the buckets in the order they were opened: a bucket holding a tail slice
  is a hybrid chunk, the others batched chunks; members in the order they
  joined.
"""

from __future__ import annotations

import math


def piece_time(ctx: int, s: int, alpha1: float, alpha2: float) -> float:
    """Eq. (1): time of one slice of s tokens after a context of ctx tokens."""
    quad = int(s) * (2 * int(ctx) + int(s))  # (ctx + s)^2 - ctx^2, exact
    return alpha1 * float(quad) + alpha2 * float(int(s))


def mesh(L: int, K: int, alpha1: float, alpha2: float) -> list[int]:
    """Boundaries 0 = b_0 < b_1 < ... < b_K = L of the longest sequence cut
    into K slices of (as nearly as integers allow) equal eq.-(1) time."""
    L, K = int(L), int(K)
    if K < 1 or L < K:
        raise ValueError("need 1 <= K <= L")
    if not (alpha1 > 0.0) or not (alpha2 >= 0.0) or math.isinf(alpha1) or math.isinf(alpha2):
        raise ValueError("need alpha1 > 0 and alpha2 >= 0, finite")

    def f(b):
        return alpha1 * float(b * b) + alpha2 * float(b)

    total = f(L)
    bounds = [0]
    for i in range(1, K):
        goal = float(i) * total
        t = goal / float(K)
        root = (-alpha2 + math.sqrt(alpha2 * alpha2 + 4.0 * alpha1 * t)) / (2.0 * alpha1)
        lo, hi = bounds[-1] + 1, L - (K - i)  # every slice keeps a token
        best, best_err = None, None
        for b in range(int(math.floor(root)) - 1, int(math.floor(root)) + 3):
            b = min(max(b, lo), hi)
            err = abs(float(K) * f(b) - goal)
            if best is None or err < best_err or (err == best_err and b < best):
                best, best_err = b, err
        bounds.append(best)
    bounds.append(L)
    return bounds


def split(lengths, bounds):
    """Cut every sequence by the mesh.  Returns (split_chunks,
    tails, shorts): split chunks and tails as (sequence, context, length),
    shorts as (sequence, length); empty sequences are dropped."""
    inner = bounds[1:-1]
    split_chunks, tails, shorts = [], [], []
    for j, L in enumerate(lengths):
        L = int(L)
        if L == 0:
            continue
        cuts = [b for b in inner if b < L]
        if not cuts:
            shorts.append((j, L))
            continue
        starts = [0] + cuts
        for a, b in zip(starts[:-1], cuts):
            split_chunks.append((j, a, b - a))
        tails.append((j, cuts[-1], L - cuts[-1]))
    return split_chunks, tails, shorts


def bucket_order(buckets):
    """Buckets in the order a short sequence tries them: tot_time /
    tot_tokens ascending (the share of long sequences in the bucket), ties
    to the bucket opened first."""
    return sorted(buckets, key=lambda b: (b["time"] / float(b["tokens"]), b["id"]))


def short_order(shorts, alpha1: float, alpha2: float):
    """Short sequences (sequence, length) by decreasing time, ties to the
    earlier sequence."""
    return sorted(shorts, key=lambda js: (-piece_time(0, js[1], alpha1, alpha2), js[0]))


def initial_time_threshold(L: int, K: int, alpha1: float, alpha2: float) -> float:
    """T_t before any loosening: the time of one mesh slice, f(L) / K."""
    return (alpha1 * float(L * L) + alpha2 * float(L)) / float(K)


def chunk(lengths, K: int, alpha1: float, alpha2: float, token_cap: int):
    """Algorithm 1 on one batch of sequence lengths.  Returns a list of
    chunks; each chunk is a dict with 'kind' ('split', 'hybrid' or
    'batched'), 'context' C and 'slices' [(sequence, q_lo, q_hi)] (rows
    of the sequence; keys [0, q_hi)), plus the final T_t and the mesh."""
    lengths = [int(x) for x in lengths]
    token_cap = int(token_cap)
    if any(x < 0 for x in lengths) or not lengths or max(lengths) == 0:
        raise ValueError("need non-negative lengths, not all zero")
    if token_cap < 1:
        raise ValueError("token_cap must be >= 1")
    L = max(lengths)
    bounds = mesh(L, min(int(K), L), alpha1, alpha2)
    K = len(bounds) - 1
    t_t = initial_time_threshold(L, K, alpha1, alpha2)
    t_m = token_cap
    split_chunks, tails, shorts = split(lengths, bounds)

    # buckets: dicts of id (opening order), time, tokens, members, tail
    buckets = []
    for j, c, s in tails:
        t = piece_time(c, s, alpha1, alpha2)
        buckets.append({"id": len(buckets), "time": t, "tokens": s, "members": [(j, c, s)], "tail": True})

    for j, n in short_order(shorts, alpha1, alpha2):
        t = piece_time(0, n, alpha1, alpha2)
        while True:
            if not buckets or min(b["tokens"] for b in buckets) + n > t_m:
                buckets.append({"id": len(buckets), "time": t, "tokens": n, "members": [(j, 0, n)], "tail": False})
                break
            placed = False
            for b in bucket_order(buckets):
                if b["time"] + t <= t_t and b["tokens"] + n <= t_m:
                    b["time"] += t
                    b["tokens"] += n
                    b["members"].append((j, 0, n))
                    placed = True
                    break
            if placed:
                break
            t_t = min(b["time"] + t for b in buckets if b["tokens"] + n <= t_m)

    chunks = []
    for j, c, s in split_chunks:
        chunks.append({"kind": "split", "context": c, "slices": [(j, c, c + s)],
                       "time": piece_time(c, s, alpha1, alpha2)})
    for b in sorted(buckets, key=lambda b: b["id"]):
        ctx = b["members"][0][1] if b["tail"] else 0
        chunks.append({"kind": "hybrid" if b["tail"] else "batched", "context": ctx,
                       "slices": [(j, c, c + s) for j, c, s in b["members"]], "time": b["time"]})
    return {"chunks": chunks, "mesh": bounds, "t_t": t_t}


def chunk_items(cu_seqlens, K: int, alpha1: float, alpha2: float, token_cap: int):
    """Work items of Algorithm 1's chunks for a packed batch: a slice
    [lo, hi) of the sequence starting at cu[j] is the item
    (cu[j], lo, hi, 0, hi).  Returns (items, chunk index of each item)."""
    cu = [int(c) for c in cu_seqlens]
    if not cu or cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0 and not decrease")
    lengths = [b - a for a, b in zip(cu, cu[1:])]
    res = chunk(lengths, K, alpha1, alpha2, token_cap)
    items, owner = [], []
    for ci, ch in enumerate(res["chunks"]):
        for j, lo, hi in ch["slices"]:
            items.append((cu[j], lo, hi, 0, hi))
            owner.append(ci)
    return items, owner
