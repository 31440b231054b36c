"""GPU: the whole path from an unpadded request. pad_segments builds the
padded tensors and the layout on the GPU (request preparation and per-segment
suffix padding, vllm-omni PR #8335, Purpose; diffusers cosmos_parallel.py,
shard_cosmos3_sequence), then selection and sparse and dense attention run
on them. The padded bytes equal the generator's, selections match the oracle
bit for bit and outputs are within the bf16 tolerance."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, note, out_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_blocks_amd")


def _segments_on_gpu(case):
    lay = case.layout
    pl, pv, sv = lay["kv_prefix_len"], lay["kv_prefix_valid"], lay["kv_suffix_valid"]

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")

    return (t(case.q[:, :lay["q_valid"]]), t(case.k[:, :pv]), t(case.v[:, :pv]),
            t(case.k[:, pl:pl + sv]), t(case.v[:, pl:pl + sv]))


@pytest.mark.parametrize("prefix,gen,bq,bk,d", [(100, 700, 64, 64, 128), (0, 700, 64, 64, 64),
                                                (37, 1000, 128, 64, 128), (130, 300, 64, 128, 64)])
def test_padded_request_through_select_and_attention(prefix, gen, bq, bk, d):
    case = synth.make_case(f"prep_gpu{prefix}_{gen}", hq=4, hkv=2, d=d, bq=bq, bk=bk,
                           prefix=prefix, gen=gen, cfg=72)
    note(f"[gpu] request prefix={prefix} gen={gen} block {bq}x{bk} d={d}")
    q, k, v, lay = bsa.pad_segments(*_segments_on_gpu(case), block_q=bq, block_k=bk)
    for got, ref in ((q, case.q), (k, case.k), (v, case.v)):
        assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), ref)
    nq, nk, p = bsa.num_blocks(lay)
    keep = bsa.keep_blocks(nk, p, 75)
    idx, cnt = bsa.select_blocks(q, k, lay, keep)
    out, lse = bsa.block_sparse_attention(q, k, v, idx, cnt, lay, return_lse=True)
    dense = bsa.dense_attention(q, k, v, lay)
    torch.cuda.synchronize()
    ridx, rcnt = oracle.select(case.layout, case.q, case.k, keep)
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    ro, rl = oracle.attend(case.layout, case.q, case.k, case.v, ridx, rcnt)
    rd, _ = oracle.dense(case.layout, case.q, case.k, case.v)
    rows = np.arange(lay["q_len"]) < gen
    for name, got, ref in (("sparse", out, ro), ("dense", dense, rd)):
        g = out_to_f64(got)
        assert_close(g[:, rows], ref[:, rows], what=name)
        assert (g[:, ~rows] == 0).all()
    gl = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.abs(gl[fin] - rl[fin]).max() < 1e-3
