"""Oracle, attention phase: softmax attention over the selected KV blocks.

Test infrastructure only (see the package docstring). fp64 arithmetic on the
exact fp64 widening of the bf16 inputs.

Semantics, each from the pages:
* non-causal full attention of generation queries over cat(prefix, gen) keys
  (diffusers ``cosmos_parallel.py``, ``cosmos3_cp_attention``, generation
  pathway);
* padded keys take no weight (same file, ``build_gen_key_mask``; the reading
  taken is exact exclusion, weight 0);
* query head h reads KV head h // G with no K/V copy (same file,
  ``_repeat_kv_heads``; vllm-omni PR #8335, Purpose: native MHA/MQA/GQA head
  mapping);
* the keys of a query row are the valid keys of the blocks listed for its
  (batch, head, query block) (vllm-omni PR #8335, Purpose: the selector's
  the block lists and their lengths per query head are what the backend runs);
* softmax scale defaults to head_dim ** -0.5 (mstar PR #927, automated
  review);
* padded query rows produce 0 and lse = -inf, as does a row with no valid key;
* causal dense attention (``dense_causal``): the understanding pathway
  attends causally to itself (diffusers ``cosmos_parallel.py``,
  ``cosmos3_cp_attention``, understanding pathway), with the causal diagonal
  aligned to the bottom right (mstar PR #927, automated review: the dense
  ragged wrapper keeps the FA3 call's bottom-right causal alignment).
"""
from __future__ import annotations

import math

import numpy as np

from .selector import valid_key_mask, valid_query_mask, widen_bf16


def _scale(layout: dict) -> float:
    s = layout.get("scale")
    if s is None or s <= 0:
        s = 1.0 / math.sqrt(layout["head_dim"])
    return float(np.float32(s))  # the library takes the scale as an fp32 value


def _softmax_rows(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float):
    """Plain softmax attention of rows q [n, D] over keys/vals [m, D] (m >= 1).
    Returns (o [n, D], lse [n])."""
    logits = scale * (q @ keys.T)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ vals) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def identity_selection(layout: dict):
    """Every KV block for every row: the 0 % sparsity case."""
    b_, hq = layout["batch"], layout["num_q_heads"]
    n_q = layout["q_len"] // layout["block_q"]
    n_k = layout["kv_len"] // layout["block_k"]
    idx = np.broadcast_to(np.arange(n_k, dtype=np.int32), (b_, hq, n_q, n_k)).copy()
    cnt = np.full((b_, hq, n_q), n_k, np.int32)
    return idx, cnt


def _selected_keys(layout, kmask, idx_row, count):
    bk = layout["block_k"]
    blocks = np.asarray(idx_row[:count], dtype=np.int64)
    if blocks.size == 0:
        return np.zeros(0, np.int64)
    u = (blocks[:, None] * bk + np.arange(bk)[None, :]).reshape(-1)
    return u[kmask[u]]


def attend(layout: dict, q_bits, k_bits, v_bits, idx, cnt):
    """Full oracle attention. Returns o [B, q_len, Hq, D] fp64 and
    lse [B, Hq, q_len] fp64 (natural log)."""
    hq, hkv = layout["num_q_heads"], layout["num_kv_heads"]
    grp = hq // hkv
    bq = layout["block_q"]
    scale = _scale(layout)
    kmask, qmask = valid_key_mask(layout), valid_query_mask(layout)
    b_, lq, _, d = q_bits.shape
    o = np.zeros((b_, lq, hq, d))
    lse = np.full((b_, hq, lq), -np.inf)
    for b in range(b_):
        for g in range(hkv):
            kg = widen_bf16(k_bits[b, :, g, :])
            vg = widen_bf16(v_bits[b, :, g, :])
            for h in range(g * grp, (g + 1) * grp):
                qh = widen_bf16(q_bits[b, :, h, :])
                for i in range(lq // bq):
                    rows = np.arange(i * bq, (i + 1) * bq)
                    rows = rows[qmask[rows]]
                    u = _selected_keys(layout, kmask, idx[b, h, i], int(cnt[b, h, i]))
                    if rows.size == 0 or u.size == 0:
                        continue
                    ob, lb = _softmax_rows(qh[rows], kg[u], vg[u], scale)
                    o[b, rows, h] = ob
                    lse[b, h, rows] = lb
    return o, lse


def attend_rows(layout: dict, q_bits, k_bits, v_bits, idx, cnt, rows):
    """Oracle attention for chosen query rows only (the full-size checks).

    ``rows`` [B, Hq, R] query-row indices. Returns o [B, Hq, R, D] and
    lse [B, Hq, R].

    Same definition as ``attend``: for row t of query block i, softmax over
    the valid keys of the blocks listed for (b, h, i). Evaluated for all R
    rows of a head at once: logits against every key of KV head h // G, then
    every key outside a row's selected valid set gets weight exactly 0 (its
    logit never enters the max, its value row is replaced by 0 so that
    nothing it holds can reach the sum).
    """
    hq, hkv = layout["num_q_heads"], layout["num_kv_heads"]
    grp = hq // hkv
    bq, bk = layout["block_q"], layout["block_k"]
    scale = _scale(layout)
    kmask, qmask = valid_key_mask(layout), valid_query_mask(layout)
    b_, _, _, d = q_bits.shape
    lk = k_bits.shape[1]
    n_k = lk // bk
    nr = rows.shape[2]
    o = np.zeros((b_, hq, nr, d))
    lse = np.full((b_, hq, nr), -np.inf)
    for b in range(b_):
        for g in range(hkv):
            kg = widen_bf16(k_bits[b, :, g, :])
            vg = np.where(kmask[:, None], widen_bf16(v_bits[b, :, g, :]), 0.0)
            for h in range(g * grp, (g + 1) * grp):
                t = rows[b, h].astype(np.int64)
                keys = np.zeros((nr, n_k), dtype=bool)
                for r in range(nr):
                    if not qmask[t[r]]:
                        continue
                    i = t[r] // bq
                    c = int(cnt[b, h, i])
                    keys[r, np.asarray(idx[b, h, i, :c], dtype=np.int64)] = True
                keys = np.repeat(keys, bk, axis=1) & kmask[None, :]
                live = keys.any(axis=1)
                if not live.any():
                    continue
                qr = widen_bf16(q_bits[b, t[live], h, :])
                sel = keys[live]
                logits = np.where(sel, scale * (qr @ kg.T), -np.inf)
                m = logits.max(axis=1, keepdims=True)
                p = np.where(sel, np.exp(logits - m), 0.0)
                l = p.sum(axis=1, keepdims=True)
                o[b, h, live] = (p @ vg) / l
                lse[b, h, live] = (m + np.log(l))[:, 0]
    return o, lse


def dense(layout: dict, q_bits, k_bits, v_bits):
    """Dense (0 % sparsity) attention: every KV block selected."""
    idx, cnt = identity_selection(layout)
    return attend(layout, q_bits, k_bits, v_bits, idx, cnt)


def key_ranks(layout: dict) -> np.ndarray:
    """Position of every key among the real keys, in key order (the prefix
    segment's real keys, then the generation segment's); -1 for padding."""
    kmask = valid_key_mask(layout)
    return np.where(kmask, np.cumsum(kmask) - 1, -1)


def dense_causal(layout: dict, q_bits, k_bits, v_bits):
    """Causal dense attention, bottom-right aligned over the real tokens.

    With n_k real keys and n_q = q_valid real query rows, real row t attends
    the real keys of rank r <= t + (n_k - n_q): the last real row sees every
    real key and each earlier row one key fewer. When n_k == n_q (a stream
    attending to itself) this is the usual causal mask r <= t. Padding is
    invisible: padded keys take no weight, padded rows give 0 and lse = -inf,
    as does a real row left with no key (n_q > n_k). Returns o [B, q_len, Hq,
    D] and lse [B, Hq, q_len] like ``attend``.
    """
    hq, hkv = layout["num_q_heads"], layout["num_kv_heads"]
    grp = hq // hkv
    scale = _scale(layout)
    qmask = valid_query_mask(layout)
    rank = key_ranks(layout)
    n_k = int((rank >= 0).sum())
    off = n_k - layout["q_valid"]
    b_, lq, _, d = q_bits.shape
    o = np.zeros((b_, lq, hq, d))
    lse = np.full((b_, hq, lq), -np.inf)
    t = np.nonzero(qmask)[0]
    allowed = (rank[None, :] >= 0) & (rank[None, :] <= t[:, None] + off)   # [rows, keys]
    live = allowed.any(axis=1)
    if not live.any():
        return o, lse
    t, allowed = t[live], allowed[live]
    for b in range(b_):
        for g in range(hkv):
            kg = widen_bf16(k_bits[b, :, g, :])
            vg = np.where((rank >= 0)[:, None], widen_bf16(v_bits[b, :, g, :]), 0.0)
            for h in range(g * grp, (g + 1) * grp):
                qh = widen_bf16(q_bits[b, t, h, :])
                logits = np.where(allowed, scale * (qh @ kg.T), -np.inf)
                m = logits.max(axis=1, keepdims=True)
                p = np.where(allowed, np.exp(logits - m), 0.0)
                l = p.sum(axis=1, keepdims=True)
                o[b, t, h] = (p @ vg) / l
                lse[b, h, t] = (m + np.log(l))[:, 0]
    return o, lse
