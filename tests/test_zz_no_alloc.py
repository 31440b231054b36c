"""GPU: attn_select_blocks_noalloc (the selector with the library's fixed
scratch array, for callers that cannot allocate) gives the same lists and
counts, bit for bit, as attn_select_blocks with a caller workspace, on two
calls in a row, the second with a smaller input (the array keeps the first
call's contents), and rejects a shape whose workspace exceeds the array
before touching the device."""
import ctypes

import numpy as np
import pytest

import synth
from gpu_util import case_to_gpu, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_blocks_amd")


def _select_both(case, keep):
    lay = case.layout
    q, k, _ = case_to_gpu(case)
    nq, nk, p = bsa.num_blocks(lay)
    b, hq = lay["batch"], lay["num_q_heads"]
    stream = torch.cuda.current_stream()
    ref_i, ref_c = bsa.select_blocks(q, k, lay, keep, stream=stream)
    # through the C ABI directly
    idx = torch.full((b, hq, nq, keep), -7, dtype=torch.int32, device="cuda:0")
    cnt = torch.full((b, hq, nq), -7, dtype=torch.int32, device="cuda:0")
    shape = bsa.make_shape(lay, q=q, k=k)
    st = bsa.lib.attn_select_blocks_noalloc(ctypes.byref(shape), ctypes.c_void_p(q.data_ptr()),
                                            ctypes.c_void_p(k.data_ptr()), keep,
                                            ctypes.c_void_p(idx.data_ptr()),
                                            ctypes.c_void_p(cnt.data_ptr()), keep,
                                            ctypes.c_void_p(stream.cuda_stream))
    assert st == 0, bsa.last_error()
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_i) and torch.equal(cnt, ref_c)
    return idx, cnt


def test_noalloc_selector_matches_the_workspace_selector_twice():
    big = synth.make_case("noalloc_big", hq=8, hkv=2, d=128, bq=64, bk=64, prefix=512, gen=20000,
                          cfg=75, dist="normal")
    small = synth.make_case("noalloc_small", hq=2, hkv=1, d=64, bq=64, bk=64, prefix=100, gen=700,
                            cfg=76, pad_fill=np.nan)
    for case, pct in ((big, 75), (small, 50)):
        nq, nk, p = bsa.num_blocks(case.layout)
        keep = bsa.keep_blocks(nk, p, pct)
        note(f"[gpu] noalloc selector {case.name} keep={keep}")
        _select_both(case, keep)
    # the binding's wrapper, once more on the first input
    nq, nk, p = bsa.num_blocks(big.layout)
    keep = bsa.keep_blocks(nk, p, 75)
    q, k, _ = case_to_gpu(big)
    a = bsa.select_blocks_noalloc(q, k, big.layout, keep)
    b = bsa.select_blocks(q, k, big.layout, keep)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_noalloc_selector_rejects_a_shape_beyond_its_array():
    case = synth.make_config("tiny")
    q, k, _ = case_to_gpu(case)
    # tiny's 64-key prefix, 64 query heads over 8 KV heads, 2048 query blocks
    lay = dict(case.layout, num_q_heads=64, num_kv_heads=8, q_len=64 * 2048, q_valid=64 * 2048,
               kv_len=64 + 64 * 2048, kv_suffix_valid=64 * 2048)
    assert bsa.query_support(lay)[0] == 0
    assert bsa.select_workspace_size(lay) > bsa.SELECT_STATIC_WORKSPACE_BYTES
    shape = bsa.make_shape(lay)
    st = bsa.lib.attn_select_blocks_noalloc(ctypes.byref(shape), ctypes.c_void_p(q.data_ptr()),
                                            ctypes.c_void_p(k.data_ptr()), 64, None, None, 64, None)
    assert st == 3 and "fixed array" in bsa.last_error()
