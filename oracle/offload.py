"""Oracle for the sequence-aware offload plan (float64).

TEST INFRASTRUCTURE ONLY (see the package docstring): the product library
never calls this module.

SPPO (Adaptive Sequence Pipeline Parallel Offloading), section 5.2
"Sequence-aware Offloading": subsequence i produces an activation volume A_i
(bytes); a ratio alpha_i of it is copied to host memory while the next
subsequence computes.  The GPU memory after stage i follows

    M_i = M_{i-1} + A_i - alpha_{i-1} A_{i-1},

and the ratios are chosen so that every stage moves the same volume,

    alpha_i A_i = M_threshold,

the volume one device-to-host transfer can move during one balanced
computation step (M_threshold / BW_D2H = T_balanced_comp).  Section 5.1 says
which tensors are moved: the backward-only activations of a subsequence; the
keys and values stay resident because later subsequences attend to them.

Readings (the pages leave these open):
  * alpha_i = min(1, M_threshold / A_i): a subsequence smaller than the
    threshold is moved whole; A_i = 0 gives alpha_i = 0.
  * M_0 = A_0 (before stage 0 nothing is resident).
"""

from __future__ import annotations


def plan_offload(act, threshold):
    """Offload ratios, memory after each stage and the peak, for activation
    volumes ``act`` (bytes per subsequence, in stage order) and the per-stage
    transfer volume ``threshold`` (bytes).  Returns (alpha, mem, peak) as
    Python floats; the arithmetic is float64 in the order written below."""
    act = [float(a) for a in act]
    th = float(threshold)
    if not act or th <= 0.0 or any(a < 0.0 for a in act):
        raise ValueError("need at least one non-negative volume and a positive threshold")
    alpha = []
    for a in act:
        alpha.append(0.0 if a == 0.0 else min(1.0, th / a))
    mem = []
    m = 0.0
    for i, a in enumerate(act):
        if i == 0:
            m = a
        else:
            moved = alpha[i - 1] * act[i - 1]
            m = m + a
            m = m - moved
        mem.append(m)
    return alpha, mem, max(mem)


def offload_rows(alpha, rows):
    """Whole rows of a subsequence of ``rows`` rows that a ratio ``alpha``
    moves: floor(alpha * rows), so the moved bytes never exceed the
    threshold (alpha < 1) or the subsequence (alpha = 1)."""
    r = int(float(alpha) * int(rows))
    return max(0, min(int(rows), r))
