"""C ABI: the library loads without a GPU, exports every function the header
declares, and rejects bad arguments on the host before touching the device.

Calls here never reach a kernel launch: every argument set fails host-side
validation. Fake device pointers are used only where validation must fail
before they could be dereferenced; the module is skipped if a GPU is visible,
so that a validation bug can never launch a kernel on them."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import block_sparse_attention_blocks_amd as bsa
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "bsattn.h")

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="host-validation tests use fake device pointers")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|size_t|attn_status|const char\*)\s+(attn_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_three_calls_and_helpers():
    names = _declared()
    for n in ("attn_select_blocks", "attn_block_sparse_fwd", "attn_dense_fwd",
              "attn_dense_causal_fwd"):
        assert n in names
    assert set(names) == set(bsa.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", bsa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(\w+)$", out, flags=re.M))
    for n in _declared():
        assert n in exported, n
        assert hasattr(bsa.lib, n)


def test_version_and_keep_blocks():
    assert re.match(r"^\d+\.\d+\.\d+$", bsa.version())
    assert bsa.lib.attn_keep_blocks(764, 8, 75) == 191
    assert bsa.lib.attn_keep_blocks(1354, 4, 75) == 339
    assert bsa.lib.attn_keep_blocks(8, 1, 50) == 4
    assert bsa.lib.attn_keep_blocks(8, 9, 50) == -1
    assert bsa.lib.attn_keep_blocks(8, 1, 101) == -1


def _layout(**kw):
    lay = dict(batch=1, num_q_heads=4, num_kv_heads=2, head_dim=128, block_q=64, block_k=64,
               q_len=256, q_valid=250, kv_prefix_len=64, kv_prefix_valid=40, kv_len=320,
               kv_suffix_valid=250, scale=None)
    lay.update(kw)
    return lay


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=3), 1),                   # Hq % Hkv != 0
    (dict(head_dim=96), 2),                     # unsupported head_dim
    (dict(block_q=32), 2),                      # unsupported geometry
    (dict(block_q=512, q_len=512), 2),
    (dict(block_k=256), 2),
    (dict(q_len=250), 1),                       # not a block multiple
    (dict(q_valid=300), 1),                     # valid > len
    (dict(kv_prefix_len=40), 1),
    (dict(kv_prefix_valid=65), 1),
    (dict(kv_len=300), 1),
    (dict(kv_suffix_valid=300), 1),
    (dict(batch=0), 1),
    (dict(scale=float("nan")), 1),
])
def test_shape_validation(kw, status):
    st, msg = bsa.query_support(_layout(**kw))
    assert st == status, msg
    assert "libbsattn" in msg and "gfx950" in msg


def test_query_support_ok():
    assert bsa.query_support(_layout())[0] == 0


FAKE = ctypes.c_void_p(1 << 40)          # never dereferenced: validation fails first
FAKE_MISALIGNED = ctypes.c_void_p((1 << 40) + 4)


def _shape(**kw):
    return ctypes.byref(bsa.make_shape(_layout(**kw)))


def test_select_argument_errors():
    L = bsa.lib
    ws = L.attn_select_workspace_size(_shape())
    assert ws > 0
    # keep below the protected prefix / above NK
    assert L.attn_select_blocks(_shape(), FAKE, FAKE, 0, FAKE, FAKE, 8, FAKE, ws, None) == 1
    assert L.attn_select_blocks(_shape(), FAKE, FAKE, 6, FAKE, FAKE, 8, FAKE, ws, None) == 1
    # row stride below keep
    assert L.attn_select_blocks(_shape(), FAKE, FAKE, 3, FAKE, FAKE, 2, FAKE, ws, None) == 1
    # workspace too small / missing / misaligned
    assert L.attn_select_blocks(_shape(), FAKE, FAKE, 3, FAKE, FAKE, 3, FAKE, ws - 1, None) == 3
    assert L.attn_select_blocks(_shape(), FAKE, FAKE, 3, FAKE, FAKE, 3, None, ws, None) == 3
    assert L.attn_select_blocks(_shape(), FAKE, FAKE, 3, FAKE, FAKE, 3,
                                ctypes.c_void_p((1 << 40) + 16), ws, None) == 3
    # null / misaligned tensors
    assert L.attn_select_blocks(_shape(), None, FAKE, 3, FAKE, FAKE, 3, FAKE, ws, None) == 1
    assert L.attn_select_blocks(_shape(), FAKE_MISALIGNED, FAKE, 3, FAKE, FAKE, 3, FAKE, ws, None) == 2
    assert L.attn_select_blocks(_shape(), FAKE, FAKE, 3, None, FAKE, 3, FAKE, ws, None) == 1
    # bad shape
    assert L.attn_select_blocks(_shape(head_dim=80), FAKE, FAKE, 3, FAKE, FAKE, 3, FAKE, ws, None) == 2
    assert "keep_blocks" not in bsa.last_error() and "head_dim" in bsa.last_error()


def test_attention_argument_errors():
    L = bsa.lib
    assert L.attn_block_sparse_fwd(_shape(), FAKE, FAKE, FAKE, None, FAKE, 4, FAKE, None, None) == 1
    assert L.attn_block_sparse_fwd(_shape(), FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, None) == 1
    assert L.attn_block_sparse_fwd(_shape(), FAKE, FAKE, None, FAKE, FAKE, 4, FAKE, None, None) == 1
    assert L.attn_dense_fwd(_shape(), FAKE, FAKE, FAKE, FAKE_MISALIGNED, None, None) == 2
    assert L.attn_dense_fwd(_shape(), FAKE, FAKE, FAKE, FAKE,
                            ctypes.c_void_p((1 << 40) + 2), None) == 1
    assert L.attn_dense_fwd(_shape(block_q=48), FAKE, FAKE, FAKE, FAKE, None, None) == 2
    assert L.attn_dense_causal_fwd(_shape(), FAKE, None, FAKE, FAKE, None, None) == 1
    assert L.attn_dense_causal_fwd(_shape(head_dim=96), FAKE, FAKE, FAKE, FAKE, None, None) == 2
    assert "attn_dense_causal_fwd" in bsa.last_error()
    s = bsa.make_shape(_layout())
    s.k_stride[1] = 260  # not a multiple of 8 elements
    assert L.attn_dense_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, None) == 2
    assert "k_stride" in bsa.last_error()


def test_selector_block_limit():
    lay = _layout(kv_len=64 * 4200, kv_suffix_valid=64 * 4200 - 64)
    st, msg = bsa.query_support(lay)
    assert st == 2 and "4096" in msg


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """Importing the binding with the library absent raises (no CPU fallback),
    also when BSATTN_LIBRARY names a file that does not exist."""
    import importlib.util
    import shutil
    monkeypatch.delenv("BSATTN_LIBRARY", raising=False)
    pkg = os.path.join(ROOT, "block_sparse_attention_blocks_amd")
    dst = tmp_path / "block_sparse_attention_blocks_amd"
    dst.mkdir()
    shutil.copy(os.path.join(pkg, "__init__.py"), dst / "__init__.py")
    spec = importlib.util.spec_from_file_location("bsa_nolib", dst / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError):
        spec.loader.exec_module(mod)
    monkeypatch.setenv("BSATTN_LIBRARY", str(tmp_path / "absent" / "libbsattn.so"))
    mod2 = importlib.util.module_from_spec(
        importlib.util.spec_from_file_location("bsa_nolib2", os.path.join(pkg, "__init__.py")))
    with pytest.raises(ImportError):
        mod2.__spec__.loader.exec_module(mod2)


def _golden_recipes():
    import json
    from conftest import GOLDEN
    return json.load(open(os.path.join(GOLDEN, "strategy_recipes.json")))["recipes"]


def test_strategy_decisions_match_the_oracle():
    """attn_strategy_is_sparse (host arithmetic) against the oracle's
    strategy on every (step, layer) of the pages' recipes."""
    import oracle
    for r in _golden_recipes():
        spec = r["sparse_layers"]
        layers = list(range(int(spec.split("-")[0]), int(spec.split("-")[1]) + 1)) if spec else []
        st = bsa.make_strategy(r["num_layers"], r["dense_steps"], layers, 75)
        got = [bsa.strategy_is_sparse(st, s, l) for s in range(r["steps"])
               for l in range(r["num_layers"])]
        ref = [oracle.strategy.is_sparse(r["num_layers"], r["dense_steps"], layers, s, l)
               for s in range(r["steps"]) for l in range(r["num_layers"])]
        assert got == ref
        assert sum(got) == r["sparse_calls"]


def test_strategy_validation_and_workspace():
    L = bsa.lib
    ok = bsa.make_strategy(36, 10, range(8, 36), 75)
    assert L.attn_strategy_is_sparse(ctypes.byref(ok), 0, 36) == -1
    assert L.attn_strategy_is_sparse(ctypes.byref(ok), -1, 0) == -1
    bad = bsa.AttnStrategy(36, 10, 1 << 40, 75)            # a layer bit past num_layers
    assert L.attn_strategy_is_sparse(ctypes.byref(bad), 12, 0) == -1
    assert L.attn_strategy_is_sparse(ctypes.byref(bsa.AttnStrategy(0, 0, 0, 75)), 0, 0) == -1
    assert L.attn_strategy_is_sparse(ctypes.byref(bsa.AttnStrategy(4, 0, 1, 101)), 0, 0) == -1
    assert L.attn_strategy_is_sparse(None, 0, 0) == -1
    lay = _layout()
    n = bsa.strategy_workspace_size(lay, ok)
    nq, nk, p = bsa.num_blocks(lay)
    keep = bsa.keep_blocks(nk, p, 75)
    rows = lay["batch"] * lay["num_q_heads"] * nq
    r256 = lambda x: (x + 255) // 256 * 256
    assert n == r256(rows * keep * 4) + r256(rows * 4) + bsa.select_workspace_size(lay)
    assert L.attn_strategy_workspace_size(_shape(head_dim=80), ctypes.byref(ok)) == 0
    assert L.attn_strategy_workspace_size(_shape(), ctypes.byref(bad)) == 0
    # a sparse call with too small a workspace fails on the host
    assert L.attn_strategy_fwd(_shape(), ctypes.byref(ok), 12, 9, FAKE, FAKE, FAKE, FAKE, None,
                               FAKE, n - 1, None) == 3
    assert L.attn_strategy_fwd(_shape(), ctypes.byref(ok), 0, 40, FAKE, FAKE, FAKE, FAKE, None,
                               FAKE, n, None) == 1
    assert "attn_strategy_fwd" in bsa.last_error()


def test_self_test_without_a_device_names_the_failure():
    """With no GPU visible the start-up check reports ATTN_ERR_DEVICE and a
    message naming itself and the library version; with one it must pass
    (the GPU suite checks that)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the GPU suite runs the self test")
    st = bsa.lib.attn_self_test()
    assert st == 5
    msg = bsa.last_error()
    assert "attn_self_test" in msg and bsa.version() in msg and "gfx950" in msg
    with pytest.raises(bsa.BsAttnError):
        bsa.self_test()


def test_binding_checks_tensor_shapes_against_the_layout():
    """The library sees only pointers and strides, so the binding refuses a
    tensor whose shape differs from what the layout implies (before touching
    the device)."""
    import synth
    lay = synth.make_case("shape_chk", hq=2, hkv=1, d=64, prefix=64, gen=448, cfg=1).layout
    b, lq, lk = lay["batch"], lay["q_len"], lay["kv_len"]
    q = torch.zeros((b, lq, 2, 64), dtype=torch.bfloat16)
    k = torch.zeros((b, lk, 1, 64), dtype=torch.bfloat16)
    short_q = torch.zeros((b, lq - 64, 2, 64), dtype=torch.bfloat16)
    long_q = torch.zeros((b, lq + 64, 2, 64), dtype=torch.bfloat16)  # extra rows are allowed
    wide_k = torch.zeros((b, lk, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        bsa.select_blocks(short_q, k, lay, 4)
    with pytest.raises(ValueError, match="shape"):
        bsa.select_blocks(q, wide_k, lay, 4)
    with pytest.raises(ValueError, match="shape"):
        bsa.dense_attention(q, k, k, lay, out=short_q)
    nq = lq // lay["block_q"]
    idx = torch.zeros((b, 2, nq - 1, 4), dtype=torch.int32)
    cnt = torch.zeros((b, 2, nq), dtype=torch.int32)
    with pytest.raises(ValueError, match="shape"):
        bsa.block_sparse_attention(q, k, k, idx, cnt, lay)
    with pytest.raises(ValueError, match="GPU"):  # right shapes, wrong device
        bsa.dense_attention(q, k, k, lay)
    with pytest.raises(ValueError, match="GPU"):
        bsa.dense_attention(long_q, k, k, lay)


def test_header_is_plain_c_and_a_c_program_links(tmp_path):
    """The boundary is a C ABI: the header compiles as C99 with gcc (no HIP or
    torch headers), and a C program linked against libbsattn.so calls the
    host-only entry points and gets the documented answers."""
    src = tmp_path / "abi_check.c"
    src.write_text(r"""
#include <stdio.h>
#include <string.h>
#include "bsattn.h"
int main(void) {
  attn_shape s;
  memset(&s, 0, sizeof s);
  s.batch = 1; s.num_q_heads = 32; s.num_kv_heads = 8; s.head_dim = 128;
  s.block_q = 64; s.block_k = 64; s.q_len = 48384; s.q_valid = 48360;
  s.kv_prefix_len = 512; s.kv_prefix_valid = 512; s.kv_len = 48896; s.kv_suffix_valid = 48360;
  for (int i = 0; i < 3; ++i) {
    const int64_t qs[3] = {48384LL * 32 * 128, 32 * 128, 128};
    const int64_t ks[3] = {48896LL * 8 * 128, 8 * 128, 128};
    s.q_stride[i] = qs[i]; s.o_stride[i] = qs[i]; s.k_stride[i] = ks[i]; s.v_stride[i] = ks[i];
  }
  printf("%d %d %d %zu %s\n", attn_keep_blocks(764, 8, 75), (int)attn_query_support(&s),
         (int)ATTN_ERR_SELF_TEST, attn_select_workspace_size(&s), attn_version());
  s.head_dim = 96;
  const int st = (int)attn_query_support(&s);  /* before attn_last_error: C leaves
                                                  the order of arguments open */
  printf("%d %s\n", st, attn_last_error());
  return 0;
}
""")
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(bsa.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-lbsattn",
                    f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    first = out[0].split()
    assert first[0] == "191" and first[1] == "0" and first[2] == "6"
    assert int(first[3]) > 0 and first[4] == bsa.version()
    assert out[1].startswith("2 attn_query_support: head_dim 96 unsupported")


def test_last_error_is_per_thread():
    """Each calling thread sees its own last failure."""
    import threading
    import synth
    good = synth.make_case("thr", hq=2, hkv=1, d=64, prefix=64, gen=448, cfg=1).layout
    bad = dict(good, head_dim=96)
    results = {}
    barrier = threading.Barrier(2)

    def run(name, lay):
        st = bsa.lib.attn_query_support(ctypes.byref(bsa.make_shape(lay)))
        barrier.wait()  # both calls done before either thread reads its message
        results[name] = (st, bsa.last_error())

    ts = [threading.Thread(target=run, args=("bad", bad)),
          threading.Thread(target=run, args=("good", good))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert results["bad"][0] == 2 and "head_dim 96" in results["bad"][1]
    assert results["good"] == (0, "")
