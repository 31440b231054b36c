"""Pins for the oracle's selection phase, each independent of the oracle's own
arithmetic: hand-worked fixtures, exact rationals, numpy's own fp32 rounding,
brute force over subsets and closed forms."""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- keep count
def test_keep_blocks_golden():
    for c in _load("keep_blocks.json")["cases"]:
        assert oracle.keep_blocks(c["nk"], c["p"], c["pct"]) == c["keep"], c["source"]


def test_keep_blocks_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.keep_blocks(4, 5, 50)
    with pytest.raises(ValueError):
        oracle.keep_blocks(4, 1, 101)


# ---------------------------------------------------------------- rn32_exact
def test_rn32_exact_matches_numpy_for_doubles():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(2000) * np.exp2(rng.integers(-140, 120, 2000)),
                         rng.standard_normal(200)])
    for x in xs:
        got = oracle.rn32_exact(Fraction(float(x)))
        assert got.view(np.uint32) == np.float32(x).view(np.uint32), x


def test_rn32_exact_ties_and_rationals():
    one = Fraction(1)
    ulp = Fraction(1, 2 ** 23)
    # halfway between 1 and 1+ulp -> 1 (even); halfway between 1+ulp and 1+2ulp -> 1+2ulp
    assert oracle.rn32_exact(one + ulp / 2) == np.float32(1.0)
    assert oracle.rn32_exact(one + ulp * 3 / 2) == np.float32(1.0 + 2 * 2 ** -23)
    # 1/3 is not a double; nearest fp32 by brute force over neighbours
    f = oracle.rn32_exact(Fraction(1, 3))
    third = Fraction(1, 3)
    for c in (np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(1))):
        assert abs(Fraction(float(f)) - third) < abs(Fraction(float(c)) - third)
    # just above a tie that a double would hide: 1 + ulp/2 + 2^-80 must round up
    assert oracle.rn32_exact(one + ulp / 2 + Fraction(1, 2 ** 80)) == np.float32(1.0 + 2 ** -23)
    assert oracle.rn32_exact(Fraction(-1, 2 ** 200)).view(np.uint32) == np.float32(-0.0).view(np.uint32)


# --------------------------------------------------------------------- pool
def test_pool_identical_rows_closed_form():
    c = synth.make_case(dist="cancel", hq=2, hkv=1, d=64, prefix=64, gen=448)
    qp, kp, nq, nk = oracle.pool(c.layout, c.q, c.k)
    rows_q = synth.bf16_bits_to_f32(c.q[0, ::64])             # one row per block
    rows_k = synth.bf16_bits_to_f32(c.k[0, ::64])
    assert np.array_equal(qp[0].transpose(1, 0, 2), rows_q)
    assert np.array_equal(kp[0].transpose(1, 0, 2), rows_k)
    assert (nq == 64).all() and (nk == 64).all()


def test_pool_integer_inputs_nearest_to_exact_mean():
    c = synth.make_case(dist="int", hq=2, hkv=1, d=64, prefix=40, gen=300, int_range=3)
    lay = c.layout
    qp, kp, nq, nk = oracle.pool(lay, c.q, c.k)
    qf = synth.bf16_bits_to_f32(c.q).astype(np.int64)
    # query blocks: rows [64i, 64i+64) limited to q_valid
    for h in range(2):
        for i in range(lay["q_len"] // 64):
            rows = [t for t in range(64 * i, 64 * i + 64) if t < lay["q_valid"]]
            assert nq[i] == len(rows)
            for dd in range(0, 64, 7):
                exact = Fraction(int(qf[0, rows, h, dd].sum()), len(rows))
                got = qp[0, h, i, dd]
                # nearest fp32, or (double rounding through fp64) one unit away at most
                nb = [np.nextafter(got, np.float32(-np.inf)), np.nextafter(got, np.float32(np.inf))]
                err = abs(Fraction(float(got)) - exact)
                if len(rows) & (len(rows) - 1) == 0:
                    assert all(err <= abs(Fraction(float(x)) - exact) for x in nb)
                else:
                    assert err <= abs(Fraction(float(nb[1])) - Fraction(float(nb[0])))
    # the partially valid prefix block averages its 40 valid keys only
    kf = synth.bf16_bits_to_f32(c.k).astype(np.int64)
    assert nk[0] == 40
    exact = Fraction(int(kf[0, :40, 0, 5].sum()), 40)
    assert abs(Fraction(float(kp[0, 0, 0, 5])) - exact) <= Fraction(1, 2 ** 20)


@pytest.mark.parametrize("fill", [float("nan"), 1.0e4, -3.0e38])
def test_pool_and_select_ignore_padding(fill):
    base = synth.make_case(hq=2, hkv=1, d=64, prefix=40, gen=300, cfg=7)
    dirty = synth.make_case(hq=2, hkv=1, d=64, prefix=40, gen=300, cfg=7, pad_fill=fill)
    a = oracle.pool(base.layout, base.q, base.k)
    b = oracle.pool(dirty.layout, dirty.q, dirty.k)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    ia, ca = oracle.select(base.layout, base.q, base.k, 3)
    ib, cb = oracle.select(dirty.layout, dirty.q, dirty.k, 3)
    assert np.array_equal(ia, ib) and np.array_equal(ca, cb)


# ------------------------------------------------------------------- scores
def _brute_scores(qp, kp):
    out = np.zeros((qp.shape[0], kp.shape[0]), np.float32)
    for i in range(qp.shape[0]):
        for j in range(kp.shape[0]):
            s = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qp[i], kp[j]))
            out[i, j] = oracle.rn32_exact(s)
    return out


@pytest.mark.parametrize("dist", ["normal", "cancel", "int"])
def test_block_scores_equal_exact_rounding(dist):
    c = synth.make_case(dist=dist, hq=2, hkv=1, d=64, prefix=64, gen=448, cfg=11)
    qp, kp, _, _ = oracle.pool(c.layout, c.q, c.k)
    for h in range(2):
        got, nfb = oracle.block_scores(qp[0, h], kp[0, 0])
        want = _brute_scores(qp[0, h], kp[0, 0])
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        if dist == "cancel":
            assert nfb > 0  # the exact fallback really ran


def test_block_scores_fallback_catches_fp64_error():
    # fp64 running sum: 2^60 + 1 - 2^60 = 0, but the exact score is 1.
    qp = np.array([[2.0 ** 30, 1.0, -(2.0 ** 30), 0.0]], np.float32)
    kp = np.array([[2.0 ** 30, 1.0, 2.0 ** 30, 0.0]], np.float32)
    got, nfb = oracle.block_scores(qp, kp)
    assert got[0, 0] == 1.0 and nfb == 1


# ---------------------------------------------------------------- selection
def _case_from_hand(fx):
    lay = dict(fx["layout"])
    d, bq, bk = lay["head_dim"], lay["block_q"], lay["block_k"]
    q = np.zeros((1, lay["q_len"], 1, d), np.uint16)
    k = np.zeros((1, lay["kv_len"], 1, d), np.uint16)
    for i, row in enumerate(fx["q_block_rows"]):
        q[0, i * bq:(i + 1) * bq, 0] = synth.to_bf16_bits(np.array(row, float))
    for j, row in enumerate(fx["k_block_rows"]):
        k[0, j * bk:(j + 1) * bk, 0] = synth.to_bf16_bits(np.array(row, float))
    return lay, q, k


def test_select_hand_worked():
    fx = _load("select_hand.json")
    lay, q, k = _case_from_hand(fx)
    qp, kp, _, _ = oracle.pool(lay, q, k)
    sc, _ = oracle.block_scores(qp[0, 0], kp[0, 0])
    assert sc[0].tolist() == fx["scores_by_hand"]
    for c in fx["cases"]:
        idx, cnt = oracle.select(lay, q, k, c["keep"], idx_row_stride=5)
        assert cnt[0, 0, 0] == len(c["idx"]), c["why"]
        assert idx[0, 0, 0, :cnt[0, 0, 0]].tolist() == c["idx"], c["why"]
        assert (idx[0, 0, 0, cnt[0, 0, 0]:] == -1).all()


def _check_certificate(scores, idx, cnt, p, keep, block_ok):
    """Top-k certificate of one row (independent of how it was produced)."""
    sel = idx[:cnt].tolist()
    assert sel == sorted(set(sel))
    forced = [j for j in range(p) if block_ok[j]]
    assert set(forced) <= set(sel)
    cand = [j for j in range(p, len(scores)) if block_ok[j]]
    assert cnt == len(forced) + min(keep - len(forced), len(cand))
    chosen = [j for j in sel if j >= p]
    rest = [j for j in cand if j not in chosen]
    assert all(block_ok[j] for j in sel)
    for a in chosen:
        for b in rest:
            assert scores[a] > scores[b] or (scores[a] == scores[b] and a < b)


@pytest.mark.parametrize("dist,kw", [("normal", {}), ("int", {"int_range": 1}),
                                     ("lowrank", {"frames": (1, 20, 24)}), ("cancel", {})])
def test_select_certificate(dist, kw):
    c = synth.make_case(dist=dist, hq=4, hkv=2, d=64, prefix=100, gen=480, cfg=5, **kw)
    lay = c.layout
    nk_blocks = lay["kv_len"] // 64
    p = lay["kv_prefix_len"] // 64
    keep = oracle.keep_blocks(nk_blocks, p, 60)
    idx, cnt, sc, _ = oracle.select(lay, c.q, c.k, keep, idx_row_stride=nk_blocks, return_scores=True)
    _, _, nq, nk = oracle.pool(lay, c.q, c.k)
    for h in range(4):
        for i in range(lay["q_len"] // 64):
            _check_certificate(sc[0, h, i], idx[0, h, i], cnt[0, h, i], p, keep, nk > 0)
            assert (idx[0, h, i, cnt[0, h, i]:] == -1).all()


def test_select_exhaustive_tiny():
    c = synth.make_config("tiny")
    lay = c.layout
    idx, cnt, sc, _ = oracle.select(lay, c.q, c.k, 4, return_scores=True)
    for h in range(2):
        for i in range(7):
            chosen = tuple(j for j in idx[0, h, i, :cnt[0, h, i]] if j >= 1)
            best, best_set = None, None
            for sub in itertools.combinations(range(1, 8), 3):
                tot = sum(Fraction(float(sc[0, h, i, j])) for j in sub)
                if best is None or tot > best or (tot == best and sub < best_set):
                    best, best_set = tot, sub
            assert chosen == best_set
            assert idx[0, h, i, 0] == 0  # the prefix block


def test_select_constructed_ties_take_lowest_indices():
    c = synth.make_case(hq=2, hkv=1, d=64, prefix=64, gen=448, cfg=3)
    # make every KV block identical: all scores tie
    row = c.k[0, 0].copy()
    c.k[0, :] = row
    idx, cnt = oracle.select(c.layout, c.q, c.k, 5)
    assert (idx[0, :, :, :] == np.array([0, 1, 2, 3, 4])).all()


def test_select_empty_prefix_block_not_forced():
    c = synth.make_case(hq=2, hkv=1, d=64, prefix=0, gen=448, cfg=4)
    lay = dict(c.layout)
    # a 64-key prefix segment with no valid key in it
    k = np.concatenate([np.zeros((1, 64, 1, 64), np.uint16), c.k], axis=1)
    lay.update(kv_prefix_len=64, kv_prefix_valid=0, kv_len=c.layout["kv_len"] + 64)
    idx, cnt = oracle.select(lay, c.q, k, 3)
    assert (cnt == 3).all() and (idx[..., :3] > 0).all()


def test_select_gqa_uses_group_kv_head():
    c = synth.make_case(hq=4, hkv=2, d=64, prefix=64, gen=448, cfg=8)
    idx, cnt = oracle.select(c.layout, c.q, c.k, 4)
    # query heads 2,3 must not change when KV head 0 changes
    k2 = c.k.copy()
    k2[0, :, 0] = synth.to_bf16_bits(np.random.default_rng(1).standard_normal((512, 64)))
    idx2, _ = oracle.select(c.layout, c.q, k2, 4)
    assert np.array_equal(idx[0, 2:], idx2[0, 2:])
