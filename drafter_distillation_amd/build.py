"""Build the gfx950 HIP library in-tree: drafter_distillation_amd/libav.so
(and the HBM probe executable drafter_distillation_amd/probe/hbm_probe).

    python -m drafter_distillation_amd.build

Compiles every source with hipcc for gfx950 only.  Packed-fp32 instructions
are disabled for all device code; floating-point contraction is off so that
the fused pass and the standalone backward evaluate each entry with the same
instruction sequence (the header promises identical gradient bits).
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libav.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["av_kernels.hip", "av_api.hip", "av_lmhead.hip"]

# Stand-alone HBM bandwidth probe (bench.py --workload hbm_probe): the access
# patterns of the fused pass without its arithmetic.
PROBE_SRC = os.path.join(PKG, "probe", "hbm_probe.hip")
PROBE_BIN = os.path.join(PKG, "probe", "hbm_probe")

# Libraries the shared library links beyond the HIP runtime (none).
LINK_FLAGS: list = []

# Per-source flags.  The kernels take no NaN input (the header puts
# non-finite logits outside the contract), so float max needs no NaN-quieting
# instructions; the host-side argument checks in av_api.hip do test for NaN
# and keep the default.
SOURCE_FLAGS = {"av_kernels.hip": ["-fno-honor-nans"]}

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Keep the per-thread register copies of a row as separate registers: the
    # pass that turns small private arrays into one vector value makes the
    # register allocator spill whole arrays to scratch in the row kernel.
    "-mllvm", "-amdgpu-promote-alloca-to-vector-limit=8",
    "-Wall",
    "-Wno-unused-result",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}")
    return res


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile the sources and link libav.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    cmds.append([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
                 "-packed-fp32-ops", "-Wall", PROBE_SRC, "-o", PROBE_BIN])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, *LINK_FLAGS, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
