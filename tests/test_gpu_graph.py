"""HIP graph capture of the library's calls.

Selection, selected-block attention with its log-sum-exp, dense attention and
causal dense attention are recorded into one torch.cuda.CUDAGraph. On these
paths the library makes no host synchronisation, allocates nothing and copies
nothing from the host, so the capture succeeds. The graph is then replayed
on fresh inputs written into its input buffers, with eager calls of the
library and host synchronisations between the replays. Every replay must
equal the same calls made eagerly on the same inputs, bit for bit: the
kernels are deterministic. The selector is captured both with a caller
workspace and in its allocation-free form."""
import pytest

import synth
from gpu_util import case_to_gpu, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bsa = pytest.importorskip("block_sparse_attention_blocks_amd")

N_SETS = 3
REPLAYS = 6


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_graph_replays_equal_eager_calls(noalloc):
    kw = dict(hq=4, hkv=2, d=128, bq=64, bk=64, prefix=100, gen=700)
    cases = [synth.make_case("graph", cfg=64, layer=s, **kw) for s in range(N_SETS)]
    lay = cases[0].layout
    sets = [case_to_gpu(c) for c in cases]
    nq, nk, p = bsa.num_blocks(lay)
    keep = bsa.keep_blocks(nk, p, 75)
    b, hq = lay["batch"], lay["num_q_heads"]
    dev = sets[0][0].device

    # Buffers the graph reads and writes (allocated before the capture).
    q, k, v = (torch.empty_like(t) for t in sets[0])
    idx = torch.empty((b, hq, nq, keep), dtype=torch.int32, device=dev)
    cnt = torch.empty((b, hq, nq), dtype=torch.int32, device=dev)
    ws = torch.empty(max(bsa.select_workspace_size(lay), 256), dtype=torch.uint8, device=dev)
    out, dense, causal = (torch.empty_like(q) for _ in range(3))

    def calls():
        if noalloc:
            bsa.select_blocks_noalloc(q, k, lay, keep, block_idx=idx, block_cnt=cnt)
        else:
            bsa.select_blocks(q, k, lay, keep, block_idx=idx, block_cnt=cnt, workspace=ws)
        _, lse = bsa.block_sparse_attention(q, k, v, idx, cnt, lay, out=out, return_lse=True)
        bsa.dense_attention(q, k, v, lay, out=dense)
        bsa.dense_attention(q, k, v, lay, causal=True, out=causal)
        return lse

    # Eager results of every input set.
    eager = []
    for s in range(N_SETS):
        for dst, src in zip((q, k, v), sets[s]):
            dst.copy_(src)
        lse = calls()
        torch.cuda.synchronize()
        eager.append([t.clone() for t in (idx, cnt, out, lse, dense, causal)])

    # Capture (the eager calls above were the warm-up), then replay. The
    # log-sum-exp buffer the binding allocates inside the capture comes from
    # the graph's own memory pool and is rewritten by every replay.
    for dst, src in zip((q, k, v), sets[0]):
        dst.copy_(src)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lse_g = calls()
    torch.cuda.synchronize()

    spare = torch.empty_like(q)
    names = ("block_idx", "block_cnt", "out", "lse", "dense", "causal")
    for r in range(REPLAYS):
        s = (r + 1) % N_SETS
        for dst, src in zip((q, k, v), sets[s]):
            dst.copy_(src)
        # eager work of the program between replays
        bsa.dense_attention(*sets[(s + 1) % N_SETS], lay, out=spare)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(names, (idx, cnt, out, lse_g, dense, causal), eager[s]):
            assert torch.equal(_bits(got), _bits(ref)), f"replay {r} (input set {s}): {name} differs"
        note(f"[gpu] graph ({'noalloc' if noalloc else 'workspace'}) replay {r} on input set {s}: "
             "bitwise equal to the eager calls")
