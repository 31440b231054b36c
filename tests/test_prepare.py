"""Request preparation (the host step before the boundary): the binding's
``pad_segments`` pads the generation queries to a block_q multiple and each
key/value segment (protected prefix, generation) on its own to a block_k
multiple, zero filled (vllm-omni PR #8335, Purpose: the shared layer owns the
request preparation and the suffix padding of a single document; diffusers
cosmos_parallel.py, shard_cosmos3_sequence: each pathway padded on its own).

The padded bytes and the layout must equal those of the seeded generator,
which lays out its padded cases independently of the binding."""
import numpy as np
import pytest
import torch

import block_sparse_attention_blocks_amd as bsa
import synth

INT_FIELDS = ("batch", "num_q_heads", "num_kv_heads", "head_dim", "block_q", "block_k", "q_len",
              "q_valid", "kv_prefix_len", "kv_prefix_valid", "kv_len", "kv_suffix_valid")

# (prefix, gen, block_q, block_k): a prefix that is not a block multiple, no
# prefix at all, generation lengths that are multiples of neither block size,
# and block_q != block_k.
CASES = [(100, 700, 64, 64), (0, 700, 64, 64), (64, 448, 64, 64), (1000, 2000, 128, 128),
         (37, 300, 128, 64), (130, 129, 64, 128)]


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def unpadded_segments(case):
    """The request as a caller holds it: generation queries and the two key /
    value segments without any padding."""
    lay = case.layout
    pl, pv, sv = lay["kv_prefix_len"], lay["kv_prefix_valid"], lay["kv_suffix_valid"]
    return (_t(case.q[:, :lay["q_valid"]]), _t(case.k[:, :pv]), _t(case.v[:, :pv]),
            _t(case.k[:, pl:pl + sv]), _t(case.v[:, pl:pl + sv]))


@pytest.mark.parametrize("prefix,gen,bq,bk", CASES)
def test_pad_segments_matches_the_generator_layout(prefix, gen, bq, bk):
    case = synth.make_case(f"prep{prefix}_{gen}", hq=4, hkv=2, d=64, bq=bq, bk=bk, prefix=prefix,
                           gen=gen, cfg=70)
    q, k, v, lay = bsa.pad_segments(*unpadded_segments(case), block_q=bq, block_k=bk)
    for f in INT_FIELDS:
        assert lay[f] == case.layout[f], f
    assert lay["scale"] is None  # the library's default head_dim ** -0.5
    for got, ref in ((q, case.q), (k, case.k), (v, case.v)):
        assert tuple(got.shape) == ref.shape
        assert np.array_equal(got.contiguous().view(torch.int16).numpy().view(np.uint16), ref)
    # the padding is zero and the real tokens sit where the layout says
    assert not q[:, gen:].float().abs().sum()
    assert not k[:, prefix:lay["kv_prefix_len"]].float().abs().sum()
    assert not k[:, lay["kv_prefix_len"] + gen:].float().abs().sum()


def test_pad_segments_scale_and_batch():
    case = synth.make_case("prep_b2", batch=2, hq=2, hkv=1, d=128, prefix=10, gen=70, cfg=71)
    q, k, v, lay = bsa.pad_segments(*unpadded_segments(case), block_q=64, block_k=64, scale=0.25)
    assert lay["scale"] == 0.25 and lay["batch"] == 2
    assert np.array_equal(k.view(torch.int16).numpy().view(np.uint16), case.k)
    shape = bsa.make_shape(lay, q=q, k=k, v=v)
    assert abs(shape.softmax_scale - 0.25) < 1e-7
    assert tuple(shape.k_stride) == tuple(k.stride()[:3])
