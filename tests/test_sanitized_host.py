"""The host side of libbsattn under address and undefined-behaviour
sanitizers, on the CPU.

_build/sanitized/libbsattn.so is the library with its host code instrumented
(device code unchanged). Two clients exercise it with the sanitizer runtime
loaded first: the C ABI test module (run in a child process that loads the
sanitized build through BSATTN_LIBRARY), and a C program built with the same
sanitizers that drives every host validation path and the device check
(tests/abi_host_check.c). A sanitizer report, a leak in the C program or a
wrong status fails the test. Like the C ABI tests, this runs only where no
GPU is visible: its fake device pointers must never reach a kernel.
"""
import importlib.util
import os
import subprocess
import sys

import pytest
import torch

from conftest import ROOT

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="host-validation tests use fake device pointers")

PKG = os.path.join(ROOT, "block_sparse_attention_blocks_amd")


def _build_module():
    spec = importlib.util.spec_from_file_location("_bsattn_build_san", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def sanitized():
    """Path of the sanitized library, rebuilt if any source is newer."""
    b = _build_module()
    srcs = [os.path.join(b.CSRC, f) for f in os.listdir(b.CSRC)] + \
        [os.path.join(b.INCLUDE, "bsattn.h")]
    if not os.path.exists(b.SANITIZED_LIB) or \
            os.path.getmtime(b.SANITIZED_LIB) < max(os.path.getmtime(s) for s in srcs):
        b.build_sanitized()
    return b.SANITIZED_LIB, b.sanitizer_runtime(), b.sanitizer_runtime_dir()


def _env(runtime, lib=None, leaks=False):
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS=f"detect_leaks={int(leaks)}:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    if lib:
        env["BSATTN_LIBRARY"] = lib
    return env


def _clean(r):
    text = r.stdout + r.stderr
    assert "Sanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]


def test_abi_module_under_sanitizers(sanitized):
    lib, runtime, _ = sanitized
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, cwd=ROOT, env=_env(runtime, lib))
    _clean(r)
    assert " passed" in r.stdout and "skipped" not in r.stdout, r.stdout[-2000:]


EXPECTED = {
    "keep": 191, "keep_bad": -1, "support": 0, "support_null": 1, "ws_positive": 1,
    "support_group": 1, "support_hd": 2, "support_qlen": 1, "support_stride": 2,
    "support_scale_default": 0, "support_scale_nan": 1, "ws_bad": 1,
    "sel_keep": 1, "sel_stride": 1, "sel_ws": 3, "sel_null": 1, "sel_device": 5,
    "noalloc_device": 5, "bs_null": 1, "bs_stride": 1, "bs_align": 2, "bs_device": 5,
    "dense_device": 5, "causal_device": 5, "self_test": 5,
    "strat_dense_step": 0, "strat_sparse": 1, "strat_dense_layer": 0, "strat_bad_layer": -1,
    "strat_null": -1, "strat_ws_positive": 1, "strat_ws_small": 3, "strat_device": 5,
    "support_again": 0,
}


def test_c_program_under_sanitizers(sanitized, tmp_path):
    lib, runtime, rtdir = sanitized
    exe = str(tmp_path / "abi_host_check")
    libdir = os.path.dirname(lib)
    subprocess.run(["/opt/rocm/llvm/bin/clang", "-std=c99", "-Wall", "-Werror", "-g",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-shared-libsan",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_host_check.c"),
                    "-o", exe, "-L", libdir, "-lbsattn", f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{rtdir}"],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=_env(runtime, leaks=True))
    _clean(r)
    got = {}
    last = []
    for line in r.stdout.splitlines():
        key, _, val = line.partition(" ")
        if key == "last":
            last.append(val)
        elif key != "version":
            got[key] = int(val)
    assert got == EXPECTED
    assert "no HIP device" in last[0] and "libbsattn" in last[0]
    assert last[1] == "[]"  # a successful call clears the message
