"""GPU: the selector's intermediate results, read back from the caller's
workspace after attn_select_blocks, against the oracle's pooling (block
means of the real rows: exact sum, one fp64 division, one fp32 rounding).

Workspace layout (each part starting at a 256-byte boundary, in this order):
pooled queries [B, Hq, NQ, D] fp64 (each an fp32 value), their norm bounds
[B, Hq, NQ] fp64, pooled keys transposed [B, Hkv, D, NK] fp32, their norm
bounds [B, Hkv, NK] fp64. The pooled vectors must equal the oracle's bit for
bit; the norm bounds must bound the pooled vectors' Euclidean norms from
above, tightly."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import case_to_gpu, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_blocks_amd")


def _r256(x):
    return (x + 255) // 256 * 256


def _workspace_parts(ws, lay):
    b, hq, hkv, d = lay["batch"], lay["num_q_heads"], lay["num_kv_heads"], lay["head_dim"]
    nq, nk, _ = bsa.num_blocks(lay)
    raw = ws.cpu().numpy()
    o_qp = 0
    o_qn = o_qp + _r256(b * hq * nq * d * 8)
    o_kpt = o_qn + _r256(b * hq * nq * 8)
    o_kn = o_kpt + _r256(b * hkv * d * nk * 4)
    end = o_kn + _r256(b * hkv * nk * 8)
    assert end == bsa.select_workspace_size(lay)
    qp = raw[o_qp:o_qp + b * hq * nq * d * 8].view(np.float64).reshape(b, hq, nq, d)
    qn = raw[o_qn:o_qn + b * hq * nq * 8].view(np.float64).reshape(b, hq, nq)
    kpt = raw[o_kpt:o_kpt + b * hkv * d * nk * 4].view(np.float32).reshape(b, hkv, d, nk)
    kn = raw[o_kn:o_kn + b * hkv * nk * 8].view(np.float64).reshape(b, hkv, nk)
    return qp, qn, kpt, kn


def _check_pool(case):
    lay = case.layout
    q, k, _ = case_to_gpu(case)
    nq, nk, p = bsa.num_blocks(lay)
    keep = bsa.keep_blocks(nk, p, case.sparsity or 50)
    ws = torch.empty(bsa.select_workspace_size(lay), dtype=torch.uint8, device="cuda:0")
    bsa.select_blocks(q, k, lay, keep, workspace=ws)
    torch.cuda.synchronize()
    qp, qn, kpt, kn = _workspace_parts(ws, lay)
    rqp, rkp, rnq, rnk = oracle.pool(lay, case.q, case.k)
    # pooled queries: fp32 values held in fp64, equal bit for bit
    assert np.array_equal(qp.astype(np.float32).astype(np.float64), qp)
    assert np.array_equal(qp.astype(np.float32).view(np.uint32), rqp.view(np.uint32))
    # pooled keys, transposed [.., D, NK]
    assert np.array_equal(kpt.transpose(0, 1, 3, 2).view(np.uint32), rkp.view(np.uint32))
    # norm bounds: never below the norm, at most a hair above it
    for bound, vec in ((qn, rqp), (kn, rkp)):
        nrm = np.sqrt((vec.astype(np.float64) ** 2).sum(axis=-1))
        assert (bound >= nrm).all()
        assert (bound <= nrm * (1 + 2.0 ** -30) + 1e-300).all()
    note(f"[gpu] {case.name}: pooled Q {qp.shape} and K {kpt.shape} bit-equal to the oracle")


def test_pooled_vectors_tiny():
    _check_pool(synth.make_config("tiny"))


@pytest.mark.parametrize("fill", [np.nan, 1e4])
def test_pooled_vectors_ignore_padding(fill):
    """Padding rows and keys hold NaN or 1e4 and real blocks end mid-block:
    the means cover the real tokens only (the block of padding alone pools
    to zero)."""
    case = synth.make_case(f"pool_pad{fill}", hq=4, hkv=2, d=128, prefix=100, gen=700, cfg=73,
                           pad_fill=fill)
    _check_pool(case)


def test_pooled_vectors_at_48k():
    _check_pool(synth.make_config("edge48k"))
