"""The list-checking build (libbsattn_checked.so, BSATTN_CHECK_LISTS=1) on the
GPU.

Block-sparse calls of that build validate every real query block's list on
the device before attention runs (vllm-omni PR #8335, Purpose: a provider
failure reaches the caller). Planted faults (an entry outside [0, NK), a
repeated block, a count outside [0, stride], a negative entry) are reported
as ATTN_ERR_INVALID_ARG naming the lowest faulty row, and the output buffer
is left untouched; a fault in a query block with no real row is not read by
attention and not reported; valid lists give output bit-identical to the
release build. The check kernel reads only the first min(count, stride)
slots of each row, so every planted fault stays in bounds.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import block_sparse_attention_blocks_amd as bsa
import synth
from gpu_util import case_to_gpu, note

pytestmark = pytest.mark.gpu

CHECKED = os.path.join(os.path.dirname(bsa.LIB_PATH), "libbsattn_checked.so")


@pytest.fixture(scope="module")
def checked():
    if not os.path.exists(CHECKED):
        pytest.fail(f"{CHECKED} is missing: build it (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(CHECKED)
    P = ctypes.c_void_p
    lib.attn_block_sparse_fwd.argtypes = [ctypes.POINTER(bsa.AttnShape), P, P, P, P, P,
                                          ctypes.c_int32, P, P, P]
    lib.attn_block_sparse_fwd.restype = ctypes.c_int32
    lib.attn_last_error.restype = ctypes.c_char_p
    return lib


@pytest.fixture(scope="module")
def case():
    note("listcheck: case hq=4 hkv=2 d=128 prefix=128 gen=1000 (16 query blocks, 18 KV blocks)")
    c = synth.make_case("listcheck", hq=4, hkv=2, d=128, prefix=128, gen=1000, sparsity=50)
    q, k, v = case_to_gpu(c)
    lay = c.layout
    nq, nk, p = bsa.num_blocks(lay)
    keep = bsa.keep_blocks(nk, p, c.sparsity)
    idx, cnt = bsa.select_blocks(q, k, lay, keep, keep + 2)
    torch.cuda.synchronize()
    return c, q, k, v, idx, cnt, nq, nk


def _call(lib, c, q, k, v, idx, cnt, out):
    shape = bsa.make_shape(c.layout, q=q, k=k, v=v, out=out)
    st = lib.attn_block_sparse_fwd(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   idx.data_ptr(), cnt.data_ptr(), idx.shape[-1], out.data_ptr(),
                                   None, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st, lib.attn_last_error().decode()


def test_valid_lists_match_the_release_build(checked, case):
    c, q, k, v, idx, cnt, nq, nk = case
    ref = bsa.block_sparse_attention(q, k, v, idx, cnt, c.layout)
    out = torch.full_like(q, 7.0)
    st, msg = _call(checked, c, q, k, v, idx, cnt, out)
    assert st == 0, msg
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def _planted(case, edit):
    c, q, k, v, idx, cnt, nq, nk = case
    bi, bc = idx.clone(), cnt.clone()
    edit(bi, bc, nk)
    return bi, bc


@pytest.mark.parametrize("name,edit,row,text", [
    ("entry_eq_nk", lambda i, c, nk: i.__setitem__((0, 1, 2, 3), nk), (0, 1, 2), "entry 3 is"),
    ("entry_far", lambda i, c, nk: i.__setitem__((0, 3, 5, 0), nk + 1000), (0, 3, 5), "outside [0,"),
    ("negative", lambda i, c, nk: i.__setitem__((0, 0, 7, 4), -3), (0, 0, 7), "entry 4 is -3"),
    ("repeat", lambda i, c, nk: i.__setitem__((0, 2, 1, 5), int(i[0, 2, 1, 1])), (0, 2, 1),
     "entry 5 repeats block"),
    ("count_high", lambda i, c, nk: c.__setitem__((0, 1, 9), i.shape[-1] + 1), (0, 1, 9), "count"),
    ("count_negative", lambda i, c, nk: c.__setitem__((0, 0, 0), -1), (0, 0, 0), "count -1"),
])
def test_faults_are_reported_and_nothing_is_written(checked, case, name, edit, row, text):
    c, q, k, v = case[:4]
    note(f"listcheck: planted fault {name} in row {row}")
    bi, bc = _planted(case, edit)
    out = torch.full_like(q, 7.0)
    st, msg = _call(checked, c, q, k, v, bi, bc, out)
    assert st == 1, msg
    assert f"(batch {row[0]}, head {row[1]}, query block {row[2]})" in msg, msg
    assert text in msg and "attn_block_sparse_fwd" in msg, msg
    assert bool((out == 7.0).all())


def test_lowest_faulty_row_is_reported(checked, case):
    c, q, k, v, idx, cnt, nq, nk = case

    def edit(i, cn, nk):
        i[0, 3, 0, 0] = nk          # row (0, 3, 0)
        i[0, 1, 4, 2] = -1          # row (0, 1, 4): lower
        i[0, 1, 6, 1] = i[0, 1, 6, 0]
    bi, bc = _planted(case, edit)
    out = torch.full_like(q, 7.0)
    st, msg = _call(checked, c, q, k, v, bi, bc, out)
    assert st == 1 and "(batch 0, head 1, query block 4)" in msg, msg


def test_padded_query_block_is_not_checked(checked, case):
    """A layout with one more query block past the real rows: a bad list in
    that block is never read, so the checked build does not report it."""
    c, q, k, v, idx, cnt, nq, nk = case
    lay = dict(c.layout, q_len=c.layout["q_len"] + c.layout["block_q"])
    q2 = torch.zeros((q.shape[0], lay["q_len"], q.shape[2], q.shape[3]), dtype=q.dtype, device=q.device)
    q2[:, :q.shape[1]] = q
    nq2, nk2, p2 = bsa.num_blocks(lay)
    assert nq2 == nq + 1 and -(-lay["q_valid"] // lay["block_q"]) < nq2
    keep = bsa.keep_blocks(nk2, p2, c.sparsity)
    i2, c2 = bsa.select_blocks(q2, k, lay, keep)
    i2[0, 0, nq2 - 1, 0] = nk2 + 9
    c2[0, 1, nq2 - 1] = -5
    torch.cuda.synchronize()

    class _C:  # the layout with the extra block, as the case object the helper reads
        layout = lay
    out = torch.empty_like(q2)
    st, msg = _call(checked, _C, q2, k, v, i2, c2, out)
    assert st == 0, msg
