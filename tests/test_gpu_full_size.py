"""GPU parity at the full workload sizes, launched as the benchmark launches
them (selector with one index row of exactly ``keep`` entries, then the
attention kernel, both on torch's current stream).

Selection is compared with the oracle for every (head, query block) bit for
bit. Attention is compared with the oracle on every real row for the 48k
edge-video workload, the dense 8k workload and the first dense and first
sparse layers of the two-stream schedule (one query head per worker process), and on sampled
query rows elsewhere (rows 0 and q_valid - 1 of
every head plus uniform draws), which the oracle computes one by one; padded
query rows must be exactly 0 everywhere.
"""
import numpy as np
import pytest

import oracle
import synth
from full_oracle import check_every_row
from gpu_util import MAX_ABS, MEAN_ABS, assert_close, case_to_gpu, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_blocks_amd")

LSE_TOL = 1e-3


def _gather_rows(out, lse, rows):
    """out [B, Lq, Hq, D], lse [B, Hq, Lq] on the GPU; rows [B, Hq, R] ->
    float64 numpy o [B, Hq, R, D] and lse [B, Hq, R]."""
    b_, _, hq, _ = out.shape
    r = torch.from_numpy(rows).to(out.device)
    bi = torch.arange(b_, device=out.device)[:, None, None]
    hi = torch.arange(hq, device=out.device)[None, :, None]
    o = out[bi, r, hi].float().cpu().numpy().astype(np.float64)
    l = lse[bi, hi, r].cpu().numpy().astype(np.float64) if lse is not None else None
    return o, l


def _check_rows(case, out, lse, idx, cnt, per_head, seed_layer=0, what="output"):
    lay = case.layout
    rows = synth.sample_rows(case, per_head, seed_layer)
    ro, rl = oracle.attend_rows(lay, case.q, case.k, case.v, idx, cnt, rows)
    go, gl = _gather_rows(out, lse, rows)
    mx, mean = assert_close(go, ro, what=what)
    assert np.array_equal(np.isfinite(gl), np.isfinite(rl))
    fin = np.isfinite(rl)
    assert np.abs(gl[fin] - rl[fin]).max() < LSE_TOL
    assert not bool(out[:, lay["q_valid"]:].ne(0).any()), f"{what}: padded rows not zero"
    note(f"[gpu] {case.name}: {what} on {rows.size} sampled rows: max-abs {mx:.3g} mean-abs {mean:.3g}")


def _select_and_compare(case, keep):
    """GPU selection in the benchmark's launch configuration vs the oracle,
    every row; returns the GPU tensors and the oracle arrays."""
    lay = case.layout
    q, k, v = case_to_gpu(case)
    nq, nk, p = bsa.num_blocks(lay)
    b, hq = lay["batch"], lay["num_q_heads"]
    idx = torch.empty((b, hq, nq, keep), dtype=torch.int32, device="cuda:0")
    cnt = torch.empty((b, hq, nq), dtype=torch.int32, device="cuda:0")
    ws = torch.empty(max(bsa.select_workspace_size(lay), 256), dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()
    bsa.select_blocks(q, k, lay, keep, keep, block_idx=idx, block_cnt=cnt, workspace=ws,
                      stream=stream)
    torch.cuda.synchronize()
    ridx, rcnt = oracle.select(lay, case.q, case.k, keep)
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    assert np.array_equal(gc, rcnt), "block counts differ"
    bad = np.argwhere((gi != ridx).any(axis=-1))
    assert bad.size == 0, f"block indices differ in {len(bad)} rows, first {bad[:3].tolist()}"
    real = (np.arange(nq) * lay["block_q"]) < lay["q_valid"]
    assert (rcnt[:, :, real] == keep).all()
    return (q, k, v, idx, cnt, stream), (ridx, rcnt)


def _run_again_bitwise(case, keep, q, k, v, idx, cnt, out, lse, stream):
    """A second selection and attention call on the same inputs must give the
    same bytes: the workgroup order (XCD remap, dispatch cohorts, the
    head-synchronous order at 720p) depends on blockIdx only."""
    lay = case.layout
    idx2, cnt2 = bsa.select_blocks(q, k, lay, keep, keep, stream=stream)
    out2, lse2 = bsa.block_sparse_attention(q, k, v, idx2, cnt2, lay, return_lse=True,
                                            stream=stream)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx) and torch.equal(cnt2, cnt), "second selection differs"
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16)), "second output differs"
    assert torch.equal(lse2.view(torch.int32), lse.view(torch.int32)), "second lse differs"


def _check_every_row(case, out, lse, idx, cnt, what):
    mx, mean, lse_err, pad_zero, lse_fin = check_every_row(
        case, np.asarray(idx), np.asarray(cnt), out.view(torch.int16).cpu().numpy().view(np.uint16),
        lse.cpu().numpy())
    note(f"[gpu] {case.name}: {what} on every real row: max-abs {mx:.3g} mean-abs {mean:.3g} "
         f"lse max-abs {lse_err:.3g}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max-abs {mx:.3g}, mean-abs {mean:.3g}"
    assert pad_zero, f"{what}: padded rows not zero"
    assert lse_fin and lse_err < LSE_TOL


@pytest.mark.timeout(900)
def test_edge48k_bench_launch():
    case = synth.make_config("edge48k")
    lay = case.layout
    nq, nk, p = bsa.num_blocks(lay)
    keep = bsa.keep_blocks(nk, p, case.sparsity)
    assert keep == 191
    note(f"[gpu] edge48k {lay} keep={keep}")
    (q, k, v, idx, cnt, stream), (ridx, rcnt) = _select_and_compare(case, keep)
    out = torch.empty_like(q)
    out, lse = bsa.block_sparse_attention(q, k, v, idx, cnt, lay, out=out, return_lse=True,
                                          stream=stream)
    torch.cuda.synchronize()
    _run_again_bitwise(case, keep, q, k, v, idx, cnt, out, lse, stream)
    _check_every_row(case, out, lse, ridx, rcnt, "sparse")


@pytest.mark.parametrize("name,keep_expected", [
    ("edge48k_256x128", 96), ("mha64_48k", 191), ("mqa48k", 191), ("edge48k_cp8", 191)])
def test_other_geometries_at_48k(name, keep_expected):
    """256x128 blocks, MHA at head_dim 64, MQA, and one GPU's share of the
    head-sharded workload (4 query heads, 1 KV head) at the 48k token shape:
    full selection bit-exact, sampled rows of every head."""
    case = synth.make_config(name)
    lay = case.layout
    nq, nk, p = bsa.num_blocks(lay)
    keep = bsa.keep_blocks(nk, p, case.sparsity)
    assert keep == keep_expected
    note(f"[gpu] {name} {lay} keep={keep}")
    (q, k, v, idx, cnt, stream), (ridx, rcnt) = _select_and_compare(case, keep)
    out, lse = bsa.block_sparse_attention(q, k, v, idx, cnt, lay, return_lse=True, stream=stream)
    torch.cuda.synchronize()
    _check_rows(case, out, lse, ridx, rcnt, 64, what=name)


@pytest.mark.timeout(600)
def test_dense8k_full_size():
    case = synth.make_config("dense8k")
    lay = case.layout
    nq, nk, p = bsa.num_blocks(lay)
    note(f"[gpu] dense8k {lay}")
    q, k, v = case_to_gpu(case)
    dense, dlse = bsa.dense_attention(q, k, v, lay, return_lse=True)
    torch.cuda.synchronize()
    ridx, rcnt = oracle.identity_selection(lay)
    _check_every_row(case, dense, dlse, ridx, rcnt, "dense")
    # 0 % sparsity through the selector: every block kept, same bytes as dense
    keep = bsa.keep_blocks(nk, p, 0)
    assert keep == nk
    idx, cnt = bsa.select_blocks(q, k, lay, keep)
    sparse = bsa.block_sparse_attention(q, k, v, idx, cnt, lay)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert torch.equal(sparse.view(torch.int16), dense.view(torch.int16))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_video720p_full_size():
    case = synth.make_config("video720p")
    lay = case.layout
    nq, nk, p = bsa.num_blocks(lay)
    keep = bsa.keep_blocks(nk, p, case.sparsity)
    assert keep == 339
    note(f"[gpu] video720p {lay} keep={keep}")
    (q, k, v, idx, cnt, stream), (ridx, rcnt) = _select_and_compare(case, keep)
    out, lse = bsa.block_sparse_attention(q, k, v, idx, cnt, lay, return_lse=True, stream=stream)
    torch.cuda.synchronize()
    _run_again_bitwise(case, keep, q, k, v, idx, cnt, out, lse, stream)
    _check_rows(case, out, lse, ridx, rcnt, 256, what="sparse")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layer", range(36))
def test_twostream_schedule_layer(layer):
    """Layer ``layer`` of the 36-layer two-stream schedule: the generation
    stream (20,000 tokens, padded to 20,096) attends to cat(understanding
    stream of 1,000 tokens padded to 1,024, generation stream); layers 0-7
    run the dense path, layers 8-35 select 75 % sparse with the understanding
    stream as the protected prefix."""
    case = synth.make_config("twostream", layer=layer)
    lay = case.layout
    nq, nk, p = bsa.num_blocks(lay)
    assert (nq, nk, p) == (157, 165, 8)
    if case.sparsity == 0:
        q, k, v = case_to_gpu(case)
        out, lse = bsa.dense_attention(q, k, v, lay, return_lse=True)
        torch.cuda.synchronize()
        ridx, rcnt = oracle.identity_selection(lay)
        what = f"dense layer {layer}"
    else:
        keep = bsa.keep_blocks(nk, p, case.sparsity)
        assert keep == 42
        (q, k, v, idx, cnt, stream), (ridx, rcnt) = _select_and_compare(case, keep)
        out, lse = bsa.block_sparse_attention(q, k, v, idx, cnt, lay, return_lse=True,
                                              stream=stream)
        torch.cuda.synchronize()
        what = f"sparse layer {layer}"
        # the protected understanding-stream blocks are in every real row
        assert (ridx[..., :p] == np.arange(p)).all(axis=-1)[rcnt > 0].all()
    if layer in (0, 8):  # the first dense and the first sparse layer: every real row
        _check_every_row(case, out, lse, ridx, rcnt, what)
    else:
        _check_rows(case, out, lse, ridx, rcnt, 32, seed_layer=layer, what=what)
