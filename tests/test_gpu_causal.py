"""GPU parity of the causal dense path (attn_dense_causal_fwd) against the
fp64 oracle's ``dense_causal``: outputs within max-abs 2e-2 and mean-abs 2e-3
over real rows, lse within 1e-3, padded rows and rows with no key exactly 0
with lse -inf."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, case_to_gpu, note, out_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_blocks_amd")

LSE_TOL = 1e-3


def _check(case, lay=None, what="causal"):
    lay = lay or case.layout
    note(f"[gpu] {case.name} causal {lay}")
    q, k, v = case_to_gpu(case)
    out, lse = bsa.dense_attention(q, k, v, lay, causal=True, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_causal(lay, case.q, case.k, case.v)
    g = out_to_f64(out)
    live = np.isfinite(rl)                                   # [B, Hq, q_len]
    rows_live = live.transpose(0, 2, 1)                      # [B, q_len, Hq]
    if rows_live.any():
        assert_close(g[rows_live], ro[rows_live], what=what)
    assert (g[~rows_live] == 0).all(), f"{what}: rows without a key are not zero"
    gl = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isfinite(gl), live)
    if live.any():
        assert np.abs(gl[live] - rl[live]).max() < LSE_TOL
    return out, lse


@pytest.mark.parametrize("name,kw", [
    ("square_d128_64", dict(cfg=51, hq=4, hkv=2, d=128, bq=64, bk=64, prefix=0, gen=300)),
    ("square_d128_128", dict(cfg=52, hq=4, hkv=1, d=128, bq=128, bk=128, prefix=0, gen=1000)),
    ("square_d64_128x64", dict(cfg=53, hq=3, hkv=1, d=64, bq=128, bk=64, prefix=0, gen=500)),
    ("square_d64_64x128", dict(cfg=54, hq=2, hkv=2, d=64, bq=64, bk=128, prefix=0, gen=777)),
    ("prefix_d128_64", dict(cfg=55, hq=4, hkv=2, d=128, bq=64, bk=64, prefix=100, gen=450)),
    ("prefix_d128_128", dict(cfg=56, batch=2, hq=4, hkv=1, d=128, bq=128, bk=128, prefix=130,
                             gen=700)),
    ("prefix_d64_64x128", dict(cfg=57, hq=2, hkv=1, d=64, bq=64, bk=128, prefix=64, gen=321)),
    ("one_token", dict(cfg=58, hq=2, hkv=1, d=64, bq=64, bk=64, prefix=0, gen=1)),
    ("square_256x128", dict(cfg=62, hq=4, hkv=2, d=128, bq=256, bk=128, prefix=0, gen=1000)),
    ("prefix_256x64_d64", dict(cfg=63, hq=2, hkv=1, d=64, bq=256, bk=64, prefix=100, gen=600)),
])
def test_causal_shapes(name, kw):
    _check(synth.make_case(name, **kw))


@pytest.mark.parametrize("fill", [float("nan"), 1.0e4])
def test_causal_padding_contents_do_not_matter(fill):
    kw = dict(cfg=59, hq=4, hkv=2, d=128, bq=64, bk=64, prefix=70, gen=250)
    a = synth.make_case("pad0", **kw)
    b = synth.make_case("padx", pad_fill=fill, **kw)
    out_a, _ = _check(a)
    out_b, _ = _check(b)
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))


@pytest.mark.parametrize("bq,bk", [(64, 64), (128, 128), (128, 64)])
def test_more_rows_than_keys(bq, bk):
    """n_q > n_k: the first rows see no key and must give 0 / lse -inf."""
    case = synth.make_case("wide", cfg=60, hq=2, hkv=1, d=128, bq=bq, bk=bk, prefix=0, gen=400)
    lay = dict(case.layout)
    lay["kv_suffix_valid"] = 230   # keys 230.. of the segment are treated as padding
    _check(case, lay, what=f"wide {bq}x{bk}")


def test_causal_twice_bitwise():
    case = synth.make_case("det", cfg=61, hq=4, hkv=2, d=128, bq=128, bk=128, prefix=0, gen=600)
    q, k, v = case_to_gpu(case)
    a = bsa.dense_attention(q, k, v, case.layout, causal=True)
    b = bsa.dense_attention(q, k, v, case.layout, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("layer", [0, 8, 35])
@pytest.mark.parametrize("block", [128, 64])
def test_understanding_stream_full_size(layer, block):
    """The understanding stream of the two-stream schedule at full size
    (1,000 tokens, 32 query / 8 KV heads, head_dim 128), every row."""
    _check(synth.make_und_case(layer, block=block), what=f"und layer {layer} block {block}")
