"""Build libgdn.so (the HIP kernels and the C ABI of include/gdn.h) for gfx950 with hipcc.

The library is built in-tree, next to this file: every .hip source is compiled to an object
file in parallel (build/ beside this file), then linked. Run `python -m gated_delta_rule_42_amd.build`.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(PKG, "build")
LIB = os.path.join(PKG, "libgdn.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: the kernels feed every accumulator to vector
    # instructions (packing, scaling, stores), which would otherwise first copy it out of AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]
# Instruction-scheduler strategy per source file, where a measured one beats the default (same
# instructions, outputs bitwise equal; only their order changes). Files not listed use the default.
# The iterative ILP scheduler takes the one-kernel forward at B1 H16 T32768 d128 from 297 to 285 us
# and the channel-wise-decay forward at B4 H16 T2048 d128 from 171 to 167 us on MI355X; on the
# other sources it is neutral or (the backward) slower.
_ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
SOURCE_FLAGS = {"gdn_fused.hip": _ILP, "gdn_kda.hip": _ILP}
_NOISE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(OBJ, exist_ok=True)
    objs = []
    jobs = []
    for src in sources():
        obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        jobs.append([_hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), ()), *extra_flags,
                     "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
