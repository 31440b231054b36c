"""Oracle, step/layer attention strategy: which attention a (denoising step,
layer) call runs, and what that call computes.

Test infrastructure only (see the package docstring).

From the pages: the attention strategy chooses dense or sparse attention
per denoising step and per layer (vllm-omni PR #8583, Purpose); its recipes
either turn every layer sparse from some step on or make only some layers
sparse (same section); the measured Cosmos3 mixed recipe runs 10 dense steps, then 28 of
the 36 generation layers sparse (same page, Test Result table); the MiniMax
H3 recipe keeps the first twenty denoising iterations dense, then runs every
one of its 50 DiT layers sparse (vllm-omni PR #8644, Purpose).

A strategy is (num_layers, dense_steps, sparse_layers, sparsity_pct): steps
before ``dense_steps`` are dense in every layer; from then on layer l is
sparse exactly when l is in ``sparse_layers``. A sparse call selects with
k = keep_blocks(NK, P, sparsity_pct) and attends over the selection; a dense
call attends over every block.
"""
from __future__ import annotations

from .attention import attend, dense
from .selector import keep_blocks, select


def is_sparse(num_layers: int, dense_steps: int, sparse_layers, step: int, layer: int) -> bool:
    """Whether the call of ``layer`` in denoising step ``step`` is sparse."""
    if not 0 <= layer < num_layers or step < 0:
        raise ValueError("layer or step out of range")
    if step < dense_steps:
        return False
    return layer in set(sparse_layers)


def layer_forward(layout, q_bits, k_bits, v_bits, num_layers, dense_steps, sparse_layers,
                  sparsity_pct, step, layer):
    """The attention the strategy runs for (step, layer): (o, lse, sparse?)."""
    if is_sparse(num_layers, dense_steps, sparse_layers, step, layer):
        nk = layout["kv_len"] // layout["block_k"]
        p = layout["kv_prefix_len"] // layout["block_k"]
        keep = keep_blocks(nk, p, sparsity_pct)
        idx, cnt = select(layout, q_bits, k_bits, keep)
        o, lse = attend(layout, q_bits, k_bits, v_bits, idx, cnt)
        return o, lse, True
    o, lse = dense(layout, q_bits, k_bits, v_bits)
    return o, lse, False
