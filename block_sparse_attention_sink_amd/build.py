"""Build libdbsa.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m block_sparse_attention_sink_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdbsa.so")
SOURCES = ["dbsa_host.hip", "k_stage1.hip", "k_stage2.hip", "k_shared.hip", "k_tables.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # No packed-FP32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
]
# Kernel files only: scores and probabilities are never NaN (masked scores are
# -inf, which stays honoured), so max/min need no NaN canonicalisation.  The
# host file keeps full IEEE semantics for its argument checks.
# The persistent item loops (prefill, shared-block Stage 2): machine-level
# loop-invariant code motion would hoist constants and addresses out of them
# and keep them live across the whole walk, which spills registers inside it.
KERNEL_FLAGS = {"k_stage1.hip": ["-fno-honor-nans", "-mllvm", "-disable-machine-licm"],
                "k_stage2.hip": ["-fno-honor-nans"],
                "k_shared.hip": ["-fno-honor-nans", "-mllvm", "-disable-machine-licm"]}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, *KERNEL_FLAGS.get(s, []), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        for cmd, err in zip(cmds, ex.map(_run, cmds)):
            if verbose and err.strip():
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
