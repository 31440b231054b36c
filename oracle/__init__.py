"""fp64 CPU oracle for selected-block attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library never calls it and shares no code with
it: the two meet only in the seeded input bytes from ``synth``.

What it computes, step by step, in the order of the method:

* ``keep_blocks``   - blocks kept per query-block row from a target sparsity;
* ``pool``          - per-block means of Q and K over valid tokens;
* ``block_scores``  - fp32 block scores (correctly rounded dot products);
* ``select``        - KV-block lists and their lengths per query head, protected
                      prefix always kept, top-k with ties to the lower index;
* ``attend``        - non-causal softmax attention over the selected blocks,
                      padded keys excluded, GQA head h -> KV head h // G;
* ``dense``         - the same with every block selected;
* ``dense_causal``  - causal dense attention, bottom-right aligned over the
                      real tokens (the understanding pathway's self-attention);
* ``strategy``      - which attention a (denoising step, layer) call runs
                      under a dense-then-sparse strategy, and that call.

Sources (web pages): vllm-omni PR #8335 "[Core] Add shared block-sparse
attention adapters with FlashAttention-4" (Purpose: selector producing
block lists with their lengths per query head, protected KV prefixes, suffix padding,
native MHA/MQA/GQA mapping; 75 % target sparsity); diffusers
``examples/cosmos3/cosmos_parallel.py`` (``_repeat_kv_heads``: query head i
pairs with KV group i // repeats; ``build_gen_key_mask``: padded und and gen
keys masked; ``cosmos3_cp_attention``: the generation pathway attends with full
attention to cat(und, gen)); mstar PR #927 (automated review: default softmax
scale head_dim**-0.5; bottom-right causal alignment of the dense pass);
``cosmos3_cp_attention`` again for the understanding pathway's causal
self-attention; vllm-omni PR #8583 (Purpose, Test Result) and PR #8644
(Purpose) for the step/layer strategy.

Parity: every function here is pinned by CPU tests against closed forms,
brute force, exact rational arithmetic and torch's fp64 SDPA; none is
"parity unpinned".
"""
from .selector import keep_blocks, valid_key_mask, valid_query_mask, pool, block_scores, \
    select, select_from_scores, rn32_exact, widen_bf16
from .attention import attend, attend_rows, dense, dense_causal, identity_selection, key_ranks
from . import strategy

__all__ = [
    "keep_blocks", "valid_key_mask", "valid_query_mask", "pool", "block_scores", "select",
    "select_from_scores", "rn32_exact", "widen_bf16", "attend", "attend_rows", "dense",
    "dense_causal", "identity_selection", "key_ranks", "strategy",
]
