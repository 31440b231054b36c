"""The pins catch plausible oracle mistakes.

Each case plants one mistake in the oracle on the CPU (by replacing one of its
functions for the duration of the test: a wrong scale, padding not excluded, a
wrong GQA head, K and V swapped, the lowest scores picked, the protected
prefix not forced, a floor for the ceiling in k, padding pooled, lse in the
wrong base, top-left causal alignment) and runs pins from
test_oracle_attend.py / test_oracle_select.py / test_oracle_causal.py against
it: at least one of them must fail. Nothing here touches a GPU."""
import numpy as np
import pytest

import oracle
import oracle.attention as OA
import oracle.selector as OS
import test_oracle_attend as TA
import test_oracle_causal as TC
import test_oracle_select as TS

ATTEND_PINS = [
    TA.test_hand_worked_two_keys,
    TA.test_dense_equals_sdpa,
    lambda: TA.test_sparse_attend_equals_sdpa_with_block_mask("gqa_ragged", dict(
        hq=4, hkv=2, d=64, prefix=100, gen=300, cfg=21)),
    TA.test_closed_forms,
    TA.test_lse_matches_logsumexp,
    TA.test_gqa_equals_mha_with_repeated_heads,
    lambda: TA.test_padding_invariance_and_unpadded_equivalence(float("nan")),
    TA.test_scale_default_is_inverse_sqrt_head_dim,
]
SELECT_PINS = [
    TS.test_keep_blocks_golden,
    TS.test_select_hand_worked,
    lambda: TS.test_select_certificate("normal", {}),
    TS.test_select_constructed_ties_take_lowest_indices,
    TS.test_pool_identical_rows_closed_form,
    TS.test_pool_integer_inputs_nearest_to_exact_mean,
    lambda: TS.test_pool_and_select_ignore_padding(float("nan")),
    lambda: TS.test_pool_and_select_ignore_padding(1.0e4),
]
CAUSAL_PINS = [
    lambda: TC.test_bottom_right_with_prefix_is_tail_of_square(None),
    TC.test_more_queries_than_keys,
    TC.test_alignment_matters,
]


def _wrap_attend(monkeypatch, fn):
    real = OA.attend

    def mutated(layout, q, k, v, idx, cnt):
        return fn(real, layout, q, k, v, idx, cnt)
    monkeypatch.setattr(OA, "attend", mutated)
    monkeypatch.setattr(oracle, "attend", mutated)


def _scale_off(mp):
    real = OA._scale
    mp.setattr(OA, "_scale", lambda layout: real(layout) * 1.01)


def _padding_kept(mp):
    mp.setattr(OA, "valid_key_mask", lambda layout: np.ones(layout["kv_len"], dtype=bool))


def _gqa_wrong_head(mp):
    # query head h reads KV head (h + 1) mod Hkv instead of h // G
    def fn(real, layout, q, k, v, idx, cnt):
        if layout["num_kv_heads"] > 1:
            k, v = np.roll(k, 1, axis=2), np.roll(v, 1, axis=2)
        else:
            q = q[:, :, ::-1]  # MQA: pair the heads with each other's lists instead
        return real(layout, q, k, v, idx, cnt)
    _wrap_attend(mp, fn)


def _k_v_swapped(mp):
    _wrap_attend(mp, lambda real, layout, q, k, v, idx, cnt: real(layout, q, v, k, idx, cnt))


def _lse_base2(mp):
    def fn(real, layout, q, k, v, idx, cnt):
        o, lse = real(layout, q, k, v, idx, cnt)
        return o, lse / np.log(2.0)
    _wrap_attend(mp, fn)


def _lowest_scores(mp):
    real = OS.select_from_scores
    mp.setattr(OS, "select_from_scores",
               lambda scores, n_protected, keep, block_ok, row_ok=True:
               real(-scores, n_protected, keep, block_ok, row_ok))


def _prefix_not_forced(mp):
    real = OS.select_from_scores
    mp.setattr(OS, "select_from_scores",
               lambda scores, n_protected, keep, block_ok, row_ok=True:
               real(scores, 0, keep, block_ok, row_ok))


def _keep_floor(mp):
    def floor_keep(n_kv_blocks, n_protected, sparsity_pct):
        k = (n_kv_blocks * (100 - sparsity_pct)) // 100
        return min(max(k, n_protected), n_kv_blocks)
    mp.setattr(OS, "keep_blocks", floor_keep)
    mp.setattr(oracle, "keep_blocks", floor_keep)


def _padding_pooled(mp):
    real = OS._pool_one
    mp.setattr(OS, "_pool_one", lambda xh, mask, block:
               real(np.nan_to_num(xh, nan=0.0, posinf=0.0, neginf=0.0), np.ones_like(mask), block))


def _causal_top_left(mp):
    real = OA.key_ranks

    def shifted(layout):
        r = real(layout)
        n_k = int((r >= 0).sum())
        # ranks pushed up by n_k - n_q: row t then sees ranks <= t (top left)
        return np.where(r >= 0, r + (n_k - layout["q_valid"]), -1)
    mp.setattr(OA, "key_ranks", shifted)


MUTATIONS = [
    ("scale off by 1 %", _scale_off, ATTEND_PINS),
    ("padded keys not excluded", _padding_kept, ATTEND_PINS),
    ("wrong KV head for a query head", _gqa_wrong_head, ATTEND_PINS),
    ("K and V swapped", _k_v_swapped, ATTEND_PINS),
    ("lse in base 2", _lse_base2, ATTEND_PINS),
    ("lowest scores selected", _lowest_scores, SELECT_PINS),
    ("protected prefix not forced", _prefix_not_forced, SELECT_PINS),
    ("k rounded down", _keep_floor, SELECT_PINS),
    ("padding rows pooled", _padding_pooled, SELECT_PINS),
    ("causal diagonal at the top left", _causal_top_left, CAUSAL_PINS),
]


@pytest.mark.parametrize("what,plant,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_a_pin_catches_the_planted_mistake(monkeypatch, what, plant, pins):
    # the pins pass on the oracle as it is (checked by their own tests); with
    # the mistake planted, at least one of them must fail
    plant(monkeypatch)
    caught = []
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught.append(getattr(pin, "__name__", "pin"))
            break
    assert caught, f"no pin caught the planted mistake: {what}"
