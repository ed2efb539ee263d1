"""Builds libsegattn.so in-tree for gfx950 with hipcc.

    python -m segmented_causal_attention_amd.build       (or build() from Python)

Every call recompiles all sources (no staleness checks): hipcc cross-compiles
for gfx950 without a GPU.  Compiler flags:
  --offload-arch=gfx950   CDNA4 code object only
  -Xclang -target-feature -Xclang -packed-fp32-ops
                          disables packed-fp32 VALU forms for the device code
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsegattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# HIP translation units (kernels, and the host layer that launches them)
HIP_SOURCES = ["fwd.hip", "bwd.hip", "bwd_dqfirst.hip", "misc.hip", "api.cpp"]
# plain C++ (no HIP headers): the integer planner
CPP_SOURCES = ["planner.cpp", "chunking.cpp"]
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wno-unused-function", "-Werror=uninitialized"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="segattn_build_") as tmp:
        cmds = [[HIPCC, *COMMON, *DEVICE_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src),
                 "-o", os.path.join(tmp, src + ".o")] for src in HIP_SOURCES]
        cmds += [[HIPCC, *COMMON, "-x", "c++", "-c", os.path.join(CSRC, src),
                  "-o", os.path.join(tmp, src + ".o")] for src in CPP_SOURCES]
        objs = [c[-1] for c in cmds]
        # one compiler process per translation unit, all at once
        with ThreadPoolExecutor(len(cmds)) as ex:
            list(ex.map(_run, cmds))
        tmp_lib = LIB + ".tmp"
        _run([HIPCC, "-shared", "-fPIC", *DEVICE_FLAGS, *objs, "-o", tmp_lib])
        os.replace(tmp_lib, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
