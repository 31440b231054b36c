"""Build libbsattn.so (HIP, gfx950) in-tree with hipcc.

Every .hip file under csrc/ is compiled to an object (in parallel) and the
objects are linked into block_sparse_attention_blocks_amd/libbsattn.so. Runs
without a GPU: hipcc cross-compiles for gfx950.

Two more builds of the same sources serve the tests:
- libbsattn_checked.so (next to the release library): BSATTN_CHECK_LISTS=1,
  block-sparse calls first validate every block list on the device;
- _build/sanitized/libbsattn.so: host code built with address and
  undefined-behaviour sanitizers (device code as usual), for the CPU tests of
  the C ABI. A process loading it must preload SANITIZER_RUNTIME.
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
CHECKED_LIB = os.path.join(PKG, "libbsattn_checked.so")
SANITIZED_DIR = os.path.join(BUILD_DIR, "sanitized")
SANITIZED_LIB = os.path.join(SANITIZED_DIR, "libbsattn.so")

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


# Host-only sanitizer flags: each -fsanitize= follows its own -Xarch_host, so
# the device code of the sanitized build is compiled exactly as in the others.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def sanitizer_runtime_dir() -> str:
    """Directory of the compiler's shared address-sanitizer runtime."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return os.path.dirname(hits[-1])


def sanitizer_runtime() -> str:
    return os.path.join(sanitizer_runtime_dir(), "libclang_rt.asan-x86_64.so")


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


def _build_one(out_lib: str, obj_dir: str, extra_flags, link_flags, verbose: bool) -> str:
    hipcc = _hipcc()
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for src in srcs:
            obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
            objs.append(obj)
            extra = FILE_FLAGS.get(os.path.basename(src), [])
            cmd = [hipcc, *HIP_FLAGS, *extra, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c", src,
                   "-o", obj]
            jobs.append((src, ex.submit(_run, cmd)))
        for src, fut in jobs:
            rc, out = fut.result()
            if verbose and out.strip():
                print(out, file=sys.stderr)
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
    tmp = out_lib + ".tmp"
    rc, out = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_flags, "-o", tmp,
                    *objs])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    os.replace(tmp, out_lib)
    return out_lib


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libbsattn.so. Returns its path."""
    return _build_one(LIB, BUILD_DIR, [], [], verbose)


def build_checked(verbose: bool = False) -> str:
    """libbsattn_checked.so: the release build plus the device check of every
    block list before block-sparse attention."""
    return _build_one(CHECKED_LIB, os.path.join(BUILD_DIR, "checked"),
                      ["-DBSATTN_CHECK_LISTS=1"], [], verbose)


def build_sanitized(verbose: bool = False) -> str:
    """_build/sanitized/libbsattn.so: host code under address and
    undefined-behaviour sanitizers (for CPU tests of the C ABI)."""
    rt = sanitizer_runtime_dir()
    return _build_one(SANITIZED_LIB, SANITIZED_DIR, SANITIZE_HOST,
                      [*SANITIZE_HOST[:4], "-shared-libsan", f"-Wl,-rpath,{rt}"], verbose)


def build_all(verbose: bool = False) -> str:
    """The release library, then the checked and sanitized test builds."""
    lib = build(verbose)
    build_checked(verbose)
    build_sanitized(verbose)
    return lib


if __name__ == "__main__":
    print(build_all(verbose=True))
