"""Oracle, selection phase: keep count, block pooling, block scores, top-k.

Test infrastructure only (see the package docstring). fp64 throughout; the
selection is an integer result, so every floating-point decision is taken on
fully specified fp32 values (the block scores) that the GPU side reproduces
exactly.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


# --------------------------------------------------------------------------- S0
def keep_blocks(n_kv_blocks: int, n_protected: int, sparsity_pct: int) -> int:
    """Blocks kept per query-block row, protected prefix blocks included.

    The pages give a *target* sparsity (75 %, vllm-omni PR #8335, Purpose) and
    a protected KV prefix that the selector always keeps (same section). Reading
    taken: the protected blocks count inside the kept budget, and the budget is
    ceil(NK * (100 - pct) / 100) clamped to [P, NK], in integer arithmetic.
    """
    if n_kv_blocks < 0 or n_protected < 0 or n_protected > n_kv_blocks:
        raise ValueError("need 0 <= n_protected <= n_kv_blocks")
    if not 0 <= sparsity_pct <= 100:
        raise ValueError("sparsity_pct must be in [0, 100]")
    k = -((-n_kv_blocks * (100 - sparsity_pct)) // 100)  # ceil without floats
    return max(n_protected, min(n_kv_blocks, k))


# ------------------------------------------------------------------ validity
def valid_key_mask(layout: dict) -> np.ndarray:
    """bool[kv_len]: key u is real iff it lies in the valid part of the
    protected prefix segment or of the generation segment. Each segment is
    padded on its own and padded keys are masked (diffusers
    ``cosmos_parallel.py``, ``shard_cosmos3_sequence`` and
    ``build_gen_key_mask``)."""
    u = np.arange(layout["kv_len"])
    pl = layout["kv_prefix_len"]
    return (u < layout["kv_prefix_valid"]) | ((u >= pl) & (u < pl + layout["kv_suffix_valid"]))


def valid_query_mask(layout: dict) -> np.ndarray:
    """bool[q_len]: query row t is real iff t < q_valid (padding rows follow)."""
    return np.arange(layout["q_len"]) < layout["q_valid"]


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64, exactly (bf16 is the top half of an fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- S1
def _check_exact_block_sums(x: np.ndarray, mask: np.ndarray):
    """The pooled mean is defined from the exact block sum. An fp64 sum of at
    most 2^8 bf16 values is exact when, inside the block, the binade span of
    the non-zero values leaves room in the 53-bit significand; refuse inputs
    outside that domain rather than return an order-dependent value."""
    a = np.where(mask[..., None], np.abs(x), 0.0)
    nz = a > 0
    if not nz.any():
        return
    _, e = np.frexp(np.where(nz, a, 1.0))
    emax = np.where(nz, e, -100000).max(axis=1)
    emin = np.where(nz, e, 100000).min(axis=1)
    n = x.shape[1]
    span = emax - emin + 8 + int(np.ceil(np.log2(max(n, 2)))) + 1
    if (np.where(emax > -100000, span, 0) > 53).any():
        raise ValueError("block values span too many binades for an exact fp64 sum")


def _pool_one(xh: np.ndarray, mask: np.ndarray, block: int):
    """xh [L, D] fp64, mask [L] -> (means fp32 [NB, D], counts [NB])."""
    length, d = xh.shape
    nb = length // block
    xb = xh.reshape(nb, block, d)
    mb = mask.reshape(nb, block)
    _check_exact_block_sums(xb, mb)
    sums = np.where(mb[..., None], xb, 0.0).sum(axis=1)       # exact (checked above)
    cnt = mb.sum(axis=1)
    safe = np.where(cnt > 0, cnt, 1).astype(np.float64)
    mean64 = sums / safe[:, None]                              # one fp64 division
    mean32 = mean64.astype(np.float32)                         # one rounding to fp32
    mean32[cnt == 0] = 0.0
    return mean32, cnt


def pool(layout: dict, q_bits: np.ndarray, k_bits: np.ndarray):
    """Mean-pool Q per (batch, query head, q-block) and K per (batch, KV head,
    KV block) over valid tokens only.

    The pages do not spell out how the selector scores blocks (vllm-omni PR
    #8335, Purpose, says only that it lists KV blocks, with their number, for
    each query head and query block). Reading taken: block-mean pooling of Q
    and K. The mean is the
    exact block sum divided once in fp64 and rounded once to fp32.

    Returns qp [B,Hq,NQ,D] fp32, kp [B,Hkv,NK,D] fp32, nq [NQ] and nk [NK]
    valid-token counts.
    """
    bq, bk = layout["block_q"], layout["block_k"]
    qmask, kmask = valid_query_mask(layout), valid_key_mask(layout)
    b_, lq, hq, d = q_bits.shape
    _, lk, hkv, _ = k_bits.shape
    qp = np.zeros((b_, hq, lq // bq, d), np.float32)
    kp = np.zeros((b_, hkv, lk // bk, d), np.float32)
    nq = nk = None
    for b in range(b_):
        for h in range(hq):
            qp[b, h], nq = _pool_one(widen_bf16(q_bits[b, :, h, :]), qmask, bq)
        for g in range(hkv):
            kp[b, g], nk = _pool_one(widen_bf16(k_bits[b, :, g, :]), kmask, bk)
    if nq is None:
        nq = valid_query_mask(layout).reshape(-1, bq).sum(axis=1)
    if nk is None:
        nk = valid_key_mask(layout).reshape(-1, bk).sum(axis=1)
    return qp, kp, nq, nk


# --------------------------------------------------------------------------- S2
_F32_MAX = Fraction(2) ** 128 - Fraction(2) ** 104
_F32_OVERFLOW = Fraction(2) ** 128 - Fraction(2) ** 103   # halfway to 2^128


def rn32_exact(x: Fraction) -> np.float32:
    """The fp32 value nearest to the rational ``x``, ties to even (IEEE RN)."""
    if x == 0:
        return np.float32(0.0)
    if abs(x) >= _F32_OVERFLOW:
        return np.float32(np.inf) if x > 0 else np.float32(-np.inf)
    f = np.float32(float(x))
    best, best_err = None, None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        c = np.float32(c)
        if not np.isfinite(c):
            continue
        err = abs(Fraction(float(c)) - x)
        if best is None or err < best_err or (
                err == best_err and (int(c.view(np.uint32)) & 1) == 0 and
                (int(best.view(np.uint32)) & 1) == 1):
            best, best_err = c, err
    if best == 0:  # keep the sign of the rounded-away value
        best = np.float32(-0.0) if x < 0 else np.float32(0.0)
    return best


def _exact_dot(a: np.ndarray, b: np.ndarray) -> Fraction:
    return sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, b)), Fraction(0))


def block_scores(qp: np.ndarray, kp: np.ndarray):
    """Score of KV block j for query block i: the fp32 value nearest to the
    exact dot product of the two fp32 pooled vectors.

    Computed as an fp64 dot product; where the rigorous error bound of that
    fp64 sum leaves the fp32 rounding undecided, the products are summed as
    exact rationals instead. Either way the result is the correctly rounded
    score, independent of summation order. No softmax scale is applied: a
    positive factor does not change the order but could merge fp32 values.

    qp [NQ, D], kp [NK, D] fp32 -> (scores [NQ, NK] fp32, number of exact fallbacks).
    """
    q64 = qp.astype(np.float64)
    k64 = kp.astype(np.float64)
    d = qp.shape[-1]
    s = q64 @ k64.T
    a = np.abs(q64) @ np.abs(k64).T
    gamma = (d + 2) * 2.0 ** -53 / (1.0 - (d + 2) * 2.0 ** -53)
    widen = 2.0 * gamma * a + np.abs(s) * 2.0 ** -52
    with np.errstate(over="ignore"):
        lo = (s - widen).astype(np.float32)
        hi = (s + widen).astype(np.float32)
        out = s.astype(np.float32)
    undecided = lo.view(np.uint32) != hi.view(np.uint32)
    for i, j in zip(*np.nonzero(undecided)):
        out[i, j] = rn32_exact(_exact_dot(qp[i], kp[j]))
    return out, int(undecided.sum())


# --------------------------------------------------------------------------- S3
def select_from_scores(scores: np.ndarray, n_protected: int, keep: int,
                       block_ok: np.ndarray, row_ok: bool = True):
    """One query-block row: protected prefix blocks j < P are always kept;
    then the best remaining blocks by (score descending, index ascending) up to
    ``keep`` blocks in total (vllm-omni PR #8335, Purpose: protected KV
    prefixes; ties go to the lower block index). Empty blocks (no valid key)
    are never selected. Returns the ascending index list."""
    nk = scores.shape[0]
    if not row_ok:
        return np.zeros(0, np.int32)
    forced = [j for j in range(min(n_protected, nk)) if block_ok[j]]
    cand = np.array([j for j in range(n_protected, nk) if block_ok[j]], dtype=np.int64)
    r = max(0, min(keep - len(forced), len(cand)))
    chosen = []
    if r > 0:
        # np.lexsort: last key is primary -> sort by -score, then by index.
        order = np.lexsort((cand, -scores[cand].astype(np.float64)))
        chosen = cand[order[:r]].tolist()
    return np.array(sorted(forced + chosen), dtype=np.int32)


def select(layout: dict, q_bits: np.ndarray, k_bits: np.ndarray, keep: int, idx_row_stride=None,
           return_scores: bool = False):
    """Per-(batch, query head, query block) KV-block indices and counts.

    Each query head selects on its own (per-query-head selection, vllm-omni PR
    #8335, Purpose) against the pooled keys of its KV head h // G (diffusers
    ``cosmos_parallel.py``, ``_repeat_kv_heads``).

    Returns idx [B,Hq,NQ,stride] int32 (ascending, unused slots -1) and
    cnt [B,Hq,NQ] int32 (and the scores and fallback count if asked).
    """
    hq, hkv = layout["num_q_heads"], layout["num_kv_heads"]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    grp = hq // hkv
    bk = layout["block_k"]
    qp, kp, nq, nk = pool(layout, q_bits, k_bits)
    b_, _, n_q, _ = qp.shape
    n_k = kp.shape[2]
    p = layout["kv_prefix_len"] // bk
    if not p <= keep <= n_k:
        raise ValueError("keep must lie in [P, NK]")
    stride = keep if idx_row_stride is None else idx_row_stride
    idx = np.full((b_, hq, n_q, stride), -1, np.int32)
    cnt = np.zeros((b_, hq, n_q), np.int32)
    all_scores = np.zeros((b_, hq, n_q, n_k), np.float32) if return_scores else None
    fallbacks = 0
    for b in range(b_):
        for h in range(hq):
            sc, nf = block_scores(qp[b, h], kp[b, h // grp])
            fallbacks += nf
            if return_scores:
                all_scores[b, h] = sc
            for i in range(n_q):
                sel = select_from_scores(sc[i], p, keep, nk > 0, bool(nq[i] > 0))
                idx[b, h, i, :len(sel)] = sel
                cnt[b, h, i] = len(sel)
    if return_scores:
        return idx, cnt, all_scores, fallbacks
    return idx, cnt
