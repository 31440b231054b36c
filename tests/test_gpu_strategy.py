"""GPU: the step/layer strategy layer (attn_strategy_fwd / attn_strategy_warmup)
makes the call its schedule names and returns exactly what that call returns,
and both agree with the oracle's strategy."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, case_to_gpu, note, out_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_blocks_amd")


def _direct(q, k, v, lay, sparse, pct):
    if not sparse:
        return bsa.dense_attention(q, k, v, lay, return_lse=True)
    nq, nk, p = bsa.num_blocks(lay)
    keep = bsa.keep_blocks(nk, p, pct)
    idx, cnt = bsa.select_blocks(q, k, lay, keep)
    return bsa.block_sparse_attention(q, k, v, idx, cnt, lay, return_lse=True)


@pytest.mark.parametrize("name,kw", [
    ("tiny", None),
    ("gqa_d128", dict(cfg=71, hq=4, hkv=2, d=128, bq=64, bk=64, prefix=100, gen=600)),
    ("b256", dict(cfg=72, hq=2, hkv=1, d=128, bq=256, bk=128, prefix=128, gen=900)),
])
def test_strategy_calls_match_direct_calls_and_oracle(name, kw):
    case = synth.make_config("tiny") if kw is None else synth.make_case(name, **kw)
    lay = case.layout
    layers, dense_steps, pct = [1, 3], 2, 50
    st = bsa.make_strategy(4, dense_steps, layers, pct)
    q, k, v = case_to_gpu(case)
    ws = torch.empty(bsa.strategy_workspace_size(lay, st), dtype=torch.uint8, device=q.device)
    bsa.strategy_warmup(q, k, v, lay, st, workspace=ws)
    rows = np.arange(lay["q_len"]) < lay["q_valid"]
    for step, layer in ((0, 1), (1, 0), (2, 0), (2, 1), (5, 3), (5, 2)):
        sparse = bsa.strategy_is_sparse(st, step, layer)
        note(f"[gpu] strategy {name} step {step} layer {layer} sparse={sparse}")
        out, lse = bsa.strategy_forward(q, k, v, lay, st, step, layer, return_lse=True,
                                        workspace=ws)
        ref, rlse = _direct(q, k, v, lay, sparse, pct)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(lse, rlse)
        ro, rl, rs = oracle.strategy.layer_forward(lay, case.q, case.k, case.v, 4, dense_steps,
                                                   layers, pct, step, layer)
        assert rs == sparse
        g = out_to_f64(out)
        assert_close(g[:, rows], ro[:, rows], what=f"strategy {name} ({step}, {layer})")


def test_strategy_on_a_two_stream_layer():
    """Layer 8 of the two-stream schedule at the first sparse step of the
    Cosmos3 mixed recipe (10 dense steps, layers 8-35 sparse) and layer 3 at
    the same step (dense): the strategy's calls equal the direct ones."""
    st = bsa.make_strategy(36, 10, range(8, 36), 75)
    for layer in (3, 8):
        case = synth.make_config("twostream", layer=layer)
        lay = case.layout
        q, k, v = case_to_gpu(case)
        out = bsa.strategy_forward(q, k, v, lay, st, 10, layer)
        ref, _ = _direct(q, k, v, lay, layer >= 8, 75)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
