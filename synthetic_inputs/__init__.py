"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only draws random tensors and
sequence lengths and names the workloads.  Both the oracle side and the HIP
side receive exactly the arrays produced here.

Recipe
------
* Tensors: ``torch.Generator(device).manual_seed(seed)``, standard normal
  float32, drawn in the order Q, K, V, dO, each of shape [T, H, d]; for bf16
  workloads each float32 draw is rounded to nearest-even bf16 (torch's
  conversion).  Small cases are drawn on the CPU; the GPU tests and the bench
  may draw on ``cuda:0`` (a different but equally seeded stream), after which
  the oracle receives host copies of the very same tensors.
* Variable-length batch: sequence lengths L = clip(round(exp(N(ln 4096,
  sigma^2))), 1, 131072) with sigma = ln 16 / z_0.995 = 1.0764 (median 4096,
  0.5% above 64K), drawn with ``numpy.random.default_rng(seed + 1)`` until
  the total reaches the token budget; the last length is cut to fit.  This
  stands in for the GitHub / CommonCrawl length distributions of InfiniPipe
  Fig. 1(b), which are not available here; no dataset item is used.
"""

from __future__ import annotations

import math

import numpy as np
import torch

# Workloads: one causal attention layer, batch 1, synthetic N(0,1) inputs.
WORKLOADS = {
    "seg1k_fp32": dict(name="S1024_H1_d64_N4_fp32_fwd", S=1024, hq=1, hkv=1, d=64, N=4,
               dtype="fp32", seed=1001, fwd_only=True),
    "seg32k": dict(name="S32768_H32_d128_N8_bf16", S=32768, hq=32, hkv=32, d=128, N=8,
               dtype="bf16", seed=1002, fwd_only=False),
    "ring128k": dict(name="S131072_H32_d128_N16_ring16384_bf16", S=131072, hq=32, hkv=32,
               d=128, N=16, block=16384, dtype="bf16", seed=1003, fwd_only=False),
    "varlen256k": dict(name="varlen262144_Hq32_Hkv8_d128_slice16384_bf16", T=262144, hq=32,
               hkv=8, d=128, max_slice=16384, dtype="bf16", seed=1004, fwd_only=False),
    "seg1m": dict(name="S1048576_H40_d128_N64_bf16", S=1048576, hq=40, hkv=40, d=128,
               N=64, dtype="bf16", seed=1005, fwd_only=False),
}

LOGNORMAL_SIGMA = math.log(16.0) / 2.5758293035489004  # ln16 / z_0.995


def gen_tensors(seed, T, hq, hkv, d, dtype="bf16", device="cpu",
                names=("q", "k", "v", "do")):
    """Draw the named tensors in the fixed order q, k, v, do (skipping none:
    a tensor that is not requested is still drawn so that the others do not
    depend on the selection)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    shapes = {"q": (T, hq, d), "k": (T, hkv, d), "v": (T, hkv, d), "do": (T, hq, d)}
    out = {}
    for nm in ("q", "k", "v", "do"):
        x = torch.randn(shapes[nm], generator=gen, dtype=torch.float32, device=device)
        if nm in names:
            out[nm] = x.to(torch.bfloat16) if dtype == "bf16" else x
        del x
    return out


def lognormal_lengths(seed, total=262144, median=4096, sigma=LOGNORMAL_SIGMA,
                      max_len=131072):
    """Sequence lengths of a packed batch (see the module docstring)."""
    rng = np.random.default_rng(int(seed) + 1)
    lens = []
    acc = 0
    while acc < total:
        L = int(np.clip(round(math.exp(rng.normal(math.log(median), sigma))), 1, max_len))
        L = min(L, total - acc)
        lens.append(L)
        acc += L
    return lens


def tail_seed(start=1004, lo=65536, hi=131072, total=262144):
    """Least seed >= start whose draw holds a sequence with lo < L <= hi."""
    s = int(start)
    while True:
        if any(lo < L <= hi for L in lognormal_lengths(s, total)):
            return s
        s += 1


def cu_seqlens(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def to_numpy_f32(t):
    """Host float32 copy of a (possibly bf16, possibly device) tensor."""
    return t.detach().to("cpu", torch.float32).numpy()
