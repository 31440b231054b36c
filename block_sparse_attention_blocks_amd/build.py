"""Build libbsattn.so (HIP, gfx950) in-tree with hipcc.

Every .hip file under csrc/ is compiled to an object (in parallel) and the
objects are linked into block_sparse_attention_blocks_amd/libbsattn.so. Runs
without a GPU: hipcc cross-compiles for gfx950.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsattn.so")

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # No packed fp32 arithmetic anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# The attention kernel never relies on NaN semantics (padded keys are masked
# by index and padded V rows are cleared), so its max reductions may skip the
# NaN quieting that IEEE max would otherwise add before each v_max3. Its MFMA
# results are consumed by vector ALU code, so they are kept in ordinary VGPRs
# (no accumulation-register round trips).
FILE_FLAGS = {"attention.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbsattn)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # The host pass warns that it does not know the packed-fp32 feature: harmless.
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops" not in line)
    return r.returncode, out


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libbsattn.so. Returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for src in srcs:
            obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
            objs.append(obj)
            extra = FILE_FLAGS.get(os.path.basename(src), [])
            cmd = [hipcc, *HIP_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
            jobs.append((src, ex.submit(_run, cmd)))
        for src, fut in jobs:
            rc, out = fut.result()
            if verbose and out.strip():
                print(out, file=sys.stderr)
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
    tmp = LIB + ".tmp"
    rc, out = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
