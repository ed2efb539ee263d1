"""Shared helpers of the GPU parity tests: error metrics and the bars of the
float parity contract (bf16 inputs, fp32 accumulation, float64 oracle)."""

import sys

import numpy as np
import torch

# O and LSE: max-abs <= 1e-2 and relative-L2 <= 5e-3; dQ/dK/dV: relative-L2 <= 1e-2.
O_MAX_ABS = 1e-2
O_REL_L2 = 5e-3
G_REL_L2 = 1e-2


def host64(t):
    return t.detach().to("cpu", torch.float64).numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def errors(got, ref):
    """(max-abs, relative-L2) over the entries where the reference is finite;
    non-finite reference entries must match exactly (e.g. LSE = -inf)."""
    g, r = host64(got), host64(ref)
    fin = np.isfinite(r)
    assert np.array_equal(g[~fin], r[~fin]), "non-finite entries differ"
    assert np.all(np.isfinite(g[fin])), "non-finite values where the reference is finite"
    d = g[fin] - r[fin]
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    den = float(np.linalg.norm(r[fin]))
    rel = float(np.linalg.norm(d)) / den if den > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_close_o(got, ref, what="O"):
    ma, rl = errors(got, ref)
    print(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert ma <= O_MAX_ABS and rl <= O_REL_L2, (what, ma, rl)


def assert_close_g(got, ref, what="grad"):
    ma, rl = errors(got, ref)
    print(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert rl <= G_REL_L2, (what, ma, rl)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def segments(bounds):
    return np.array([[0, bounds[i], bounds[i + 1], 0, bounds[i + 1]] for i in range(len(bounds) - 1)], np.int64)


def ring_steps(items):
    """Group ring items by arrival step (s-th block of every segment)."""
    by = {}
    order = []
    for it in np.asarray(items).tolist():
        key = tuple(it[:3])
        if key not in by:
            by[key] = []
            order.append(key)
        by[key].append(it)
    steps = []
    s = 0
    while True:
        st = [by[k][s] for k in order if len(by[k]) > s]
        if not st:
            return steps
        steps.append(np.array(st, np.int64))
        s += 1


class Progress:
    """Progress callback for the oracle's long loops: prints the rows done
    at most every `every_s` seconds (a full-size oracle head runs for
    minutes)."""

    def __init__(self, what, every_s=20.0):
        import time
        self.what, self.every, self.t0 = what, every_s, time.perf_counter()
        self.last = self.t0

    def __call__(self, done, total):
        import time
        now = time.perf_counter()
        if now - self.last >= self.every or done == total:
            self.last = now
            say(f"  {self.what}: {done}/{total} rows, {now - self.t0:.0f} s")
