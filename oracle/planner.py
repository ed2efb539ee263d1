"""Exact-integer oracle for the host planner: FLOPs-balanced segment
boundaries, variable-length slicing and ring-order work items.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product library
never calls this module.

Work items are 5-tuples ``(seq_off, q_lo, q_hi, k_lo, k_hi)``: the query rows
``[q_lo, q_hi)`` and the key rows ``[k_lo, k_hi)`` of the packed sequence that
starts at token ``seq_off`` (sequence-local, half-open).  A query row ``q``
sees key ``k`` of an item iff ``k_lo <= k < k_hi`` and ``k <= q``.

All arithmetic uses Python integers (unbounded), so nothing here rounds.
"""

from __future__ import annotations


def tri(x: int) -> int:
    """Number of visible (query, key) pairs of a causal prefix of length x,
    diagonal included: T(x) = x(x+1)/2.

    SPPO (Adaptive Sequence Pipeline Parallel Offloading), section 3.2: under
    the causal mask the attention work of a token grows with its position; a
    token at sequence position p attends to p+1 keys.
    """
    x = int(x)
    return x * (x + 1) // 2


def segment_work(bounds):
    """Causal attention work of each segment, counted in visible pairs:
    W_i = T(b_{i+1}) - T(b_i) (query rows of segment i against the resident
    prefix 0..b_{i+1}).  InfiniPipe, section III-A2, eq. (1): the quadratic
    term (C+s)^2 - C^2 of a slice s with context C."""
    return [tri(bounds[i + 1]) - tri(bounds[i]) for i in range(len(bounds) - 1)]


def _least_b_reaching(target_times_n: int, n: int, S: int) -> int:
    """Smallest integer b in [0, S] with n*T(b) >= target_times_n (T is
    strictly increasing on b >= 0, so plain bisection is exact)."""
    lo, hi = 0, S
    while lo < hi:
        mid = (lo + hi) // 2
        if n * tri(mid) >= target_times_n:
            hi = mid
        else:
            lo = mid + 1
    return lo


def boundary(i: int, N: int, S: int) -> int:
    """Inner boundary i of the N-way partition of S tokens: the integer b in
    [0, S] minimising |N*T(b) - i*T(S)| (ties to the smaller b)."""
    goal = i * tri(S)  # compare N*T(b) against i*T(S) without division
    b = _least_b_reaching(goal, N, S)
    if b > 0 and abs(N * tri(b - 1) - goal) <= abs(N * tri(b) - goal):
        return b - 1
    return b


def partition(S: int, N: int) -> list[int]:
    """FLOPs-balanced partition of one causal sequence of length S into N
    segments; returns the boundaries b_0 = 0 < b_1 < ... < b_N = S.

    Definition (SPPO section 3.2 "FLOPs-based policy ... consistent
    computational load across subsequences" and "start with longer
    subsequences and gradually transition to shorter ones"; SPPO section 5.2
    "FLOPs-optimized subsequence partition"; InfiniPipe eq. (1) quadratic
    term): every inner boundary is the integer b minimising
    |N * T(b) - i * T(S)|, i.e. the prefix work T(b_i) is as close as an
    integer boundary allows to i/N of the total work T(S).  Ties go to the
    smaller b.  The pages write "s0 <= s1 <= ... <= sN"; this reads it as the
    boundaries increasing, which makes the segment *lengths* non-increasing.

    Raises ValueError if N < 1, S < N, or any segment would be empty.
    """
    S = int(S)
    N = int(N)
    if N < 1:
        raise ValueError("N must be >= 1")
    if S < N:
        raise ValueError("S must be >= N")
    bounds = [0] + [boundary(i, N, S) for i in range(1, N)] + [S]
    for i in range(N):
        if bounds[i + 1] <= bounds[i]:
            raise ValueError(f"empty segment {i} for S={S}, N={N}")
    return bounds


def partition_varlen(cu_seqlens, max_slice: int):
    """Work items for a packed variable-length batch (InfiniPipe section II-B:
    packed [sum(S), D] layout; section III-A1: a long sequence becomes a
    split chunk whose slices keep a context C of all earlier tokens).

    Rule (the plainest reading of "sequences longer than max_slice are split
    into FLOPs-balanced slices"; the slice cap is SPPO section 6.1's 2K-16K
    tokens per layer per device): a sequence of length L <= max_slice is one
    item attending to itself.  A longer one is cut with ``partition(L, n)``
    for the least n >= 2 whose first (longest) slice is <= max_slice; each
    slice [lo, hi) becomes an item with keys [0, hi).  Empty sequences give
    no item.  Only the chosen cut has to be free of empty slices.
    """
    max_slice = int(max_slice)
    if max_slice < 1:
        raise ValueError("max_slice must be >= 1")
    cu = [int(c) for c in cu_seqlens]
    if len(cu) < 1 or cu[0] != 0:
        raise ValueError("cu_seqlens must start at 0")
    items = []
    for s in range(len(cu) - 1):
        off, L = cu[s], cu[s + 1] - cu[s]
        if L < 0:
            raise ValueError("cu_seqlens must be non-decreasing")
        if L == 0:
            continue
        if L <= max_slice:
            items.append((off, 0, L, 0, L))
            continue
        n = 2
        while boundary(1, n, L) > max_slice:  # first (longest) slice too long
            n += 1
            if n > L:
                raise ValueError(f"cannot slice a sequence of length {L}")
        b = partition(L, n)  # raises if a slice of this cut is empty
        for i in range(n):
            items.append((off, b[i], b[i + 1], 0, b[i + 1]))
    return items


def ring_items(bounds, block: int, seq_off: int = 0):
    """Items of the ring schedule: segment i's queries [b_i, b_{i+1}) meet
    the resident K/V prefix in blocks of ``block`` tokens that arrive one
    after another, its own (diagonal) block first and then the earlier
    blocks in descending order.

    InfiniPipe section II-A: ring-style sequence parallelism runs a
    multi-step online self-attention while K/V of other slices arrive by
    point-to-point exchange.  "Sequence Parallelism" blog, Ring
    Self-Attention: device n first uses its own K^n, then receives K^{n-1},
    and so on around the ring.
    """
    block = int(block)
    if block < 1:
        raise ValueError("block must be >= 1")
    items = []
    for i in range(len(bounds) - 1):
        lo, hi = int(bounds[i]), int(bounds[i + 1])
        nblk = -(-hi // block)
        for j in range(nblk - 1, -1, -1):
            items.append((seq_off, lo, hi, j * block, min((j + 1) * block, hi)))
    return items


def ring_steps(items):
    """Group ring items by arrival step: step s holds the s-th block of every
    segment that has one.  Items of one step have disjoint query rows."""
    by_q = {}
    order = []
    for it in items:
        key = (it[0], it[1], it[2])
        if key not in by_q:
            by_q[key] = []
            order.append(key)
        by_q[key].append(it)
    steps = []
    s = 0
    while True:
        step = [by_q[k][s] for k in order if len(by_q[k]) > s]
        if not step:
            break
        steps.append(step)
        s += 1
    return steps
