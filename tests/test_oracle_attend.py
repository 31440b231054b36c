"""Pins for the oracle's attention phase: torch's fp64 SDPA on the CPU (a
library routine), closed forms, a hand-worked fixture and invariances."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import GOLDEN


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _sdpa_masked(case, idx, cnt):
    """torch SDPA (fp64, CPU) with a boolean token mask built from the block
    lists and the padding, GQA by explicit repetition of K/V heads."""
    lay = case.layout
    hq, hkv = lay["num_q_heads"], lay["num_kv_heads"]
    bq, bk = lay["block_q"], lay["block_k"]
    q = torch.from_numpy(_f64(case.q)).permute(0, 2, 1, 3)              # B,H,L,D
    k = torch.from_numpy(_f64(case.k)).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
    v = torch.from_numpy(_f64(case.v)).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
    b_, lq, lk = q.shape[0], q.shape[2], k.shape[2]
    pl = lay["kv_prefix_len"]
    key_ok = torch.zeros(lk, dtype=torch.bool)
    key_ok[:lay["kv_prefix_valid"]] = True
    key_ok[pl:pl + lay["kv_suffix_valid"]] = True
    mask = torch.zeros(b_, hq, lq, lk, dtype=torch.bool)
    for b in range(b_):
        for h in range(hq):
            for i in range(lq // bq):
                for j in idx[b, h, i, :cnt[b, h, i]]:
                    mask[b, h, i * bq:(i + 1) * bq, j * bk:(j + 1) * bk] = True
    mask &= key_ok
    rows_ok = mask.any(-1)
    safe = mask | ~rows_ok[..., None]   # rows with no key: any mask, zeroed below
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=safe,
                                                         scale=float(np.float32(lay["scale"])))
    o = torch.where(rows_ok[..., None], o, torch.zeros_like(o))
    o[:, :, lay["q_valid"]:] = 0
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("name,kw", [
    ("tiny", dict()),
    ("gqa_ragged", dict(hq=4, hkv=2, d=64, prefix=100, gen=300, cfg=21)),
    ("mqa_bq128", dict(hq=3, hkv=1, d=64, bq=128, bk=64, prefix=0, gen=500, cfg=22)),
    ("lowrank", dict(hq=4, hkv=1, d=128, prefix=64, gen=480, frames=(1, 20, 24), dist="lowrank", cfg=23)),
    ("bq256_bk128", dict(hq=2, hkv=1, d=64, bq=256, bk=128, prefix=128, gen=600, cfg=24)),
])
def test_sparse_attend_equals_sdpa_with_block_mask(name, kw):
    case = synth.make_config("tiny") if name == "tiny" else synth.make_case(**kw)
    lay = case.layout
    nk = lay["kv_len"] // lay["block_k"]
    keep = oracle.keep_blocks(nk, lay["kv_prefix_len"] // lay["block_k"], 50)
    idx, cnt = oracle.select(lay, case.q, case.k, keep)
    o, lse = oracle.attend(lay, case.q, case.k, case.v, idx, cnt)
    ref = _sdpa_masked(case, idx, cnt)
    assert np.abs(o - ref).max() < 1e-12


def test_dense_equals_sdpa():
    case = synth.make_case(hq=4, hkv=2, d=64, prefix=100, gen=300, cfg=24)
    idx, cnt = oracle.identity_selection(case.layout)
    o, _ = oracle.dense(case.layout, case.q, case.k, case.v)
    assert np.abs(o - _sdpa_masked(case, idx, cnt)).max() < 1e-12


def test_all_blocks_selected_equals_dense_and_order_free():
    case = synth.make_case(hq=2, hkv=1, d=64, prefix=64, gen=448, cfg=25)
    lay = case.layout
    nk = lay["kv_len"] // 64
    idx, cnt = oracle.select(lay, case.q, case.k, nk)     # 0 % sparsity via the selector
    o1, l1 = oracle.attend(lay, case.q, case.k, case.v, idx, cnt)
    o2, l2 = oracle.dense(lay, case.q, case.k, case.v)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12
    rng = np.random.default_rng(0)
    perm = idx.copy()
    for b, h, i in np.ndindex(*cnt.shape):
        perm[b, h, i, :cnt[b, h, i]] = rng.permutation(idx[b, h, i, :cnt[b, h, i]])
    o3, _ = oracle.attend(lay, case.q, case.k, case.v, perm, cnt)
    assert np.abs(o3 - o1).max() < 1e-12


def test_lse_matches_logsumexp():
    from scipy.special import logsumexp
    case = synth.make_config("tiny")
    lay = case.layout
    idx, cnt = oracle.select(lay, case.q, case.k, 4)
    _, lse = oracle.attend(lay, case.q, case.k, case.v, idx, cnt)
    q, k = _f64(case.q), _f64(case.k)
    for h, t in [(0, 0), (1, 200), (0, 447)]:
        i = t // 64
        keys = np.concatenate([np.arange(j * 64, j * 64 + 64) for j in idx[0, h, i, :cnt[0, h, i]]])
        logits = 0.125 * (k[0, keys, 0] @ q[0, t, h])
        assert abs(lse[0, h, t] - logsumexp(logits)) < 1e-12


def test_gqa_equals_mha_with_repeated_heads():
    case = synth.make_case(hq=4, hkv=2, d=64, prefix=64, gen=256, cfg=26)
    lay = case.layout
    idx, cnt = oracle.select(lay, case.q, case.k, 3)
    o, _ = oracle.attend(lay, case.q, case.k, case.v, idx, cnt)
    lay2 = dict(lay, num_kv_heads=4)
    k2 = np.repeat(case.k, 2, axis=2)
    v2 = np.repeat(case.v, 2, axis=2)
    o2, _ = oracle.attend(lay2, case.q, k2, v2, idx, cnt)
    assert np.array_equal(o, o2)


def test_closed_forms():
    case = synth.make_case(hq=2, hkv=1, d=64, prefix=100, gen=300, cfg=27)
    lay = case.layout
    idx, cnt = oracle.select(lay, case.q, case.k, 3)
    kmask = oracle.valid_key_mask(lay)
    v = _f64(case.v)
    # Q = 0: uniform weights -> mean of the selected valid V rows
    q0 = np.zeros_like(case.q)
    o, _ = oracle.attend(lay, q0, case.k, case.v, idx, cnt)
    for h, t in [(0, 0), (1, 299), (0, 150)]:
        i = t // 64
        keys = np.concatenate([np.arange(j * 64, j * 64 + 64) for j in idx[0, h, i, :cnt[0, h, i]]])
        keys = keys[kmask[keys]]
        assert np.abs(o[0, t, h] - v[0, keys, 0].mean(axis=0)).max() < 1e-12
    # constant V -> that constant
    vc = np.full_like(case.v, synth.to_bf16_bits(np.float64(0.75)))
    o, _ = oracle.attend(lay, case.q, case.k, vc, idx, cnt)
    assert np.abs(o[0, :300] - 0.75).max() < 1e-12
    assert (o[0, 300:] == 0).all()


def test_single_valid_key_gives_its_value():
    case = synth.make_case(hq=2, hkv=1, d=64, prefix=0, gen=1, bq=64, bk=64, cfg=28)
    lay = case.layout
    idx, cnt = oracle.identity_selection(lay)
    o, lse = oracle.attend(lay, case.q, case.k, case.v, idx, cnt)
    assert np.array_equal(o[0, 0, 0], _f64(case.v[0, 0, 0]))
    assert (o[0, 1:] == 0).all() and np.isinf(lse[0, :, 1:]).all()


def test_hand_worked_two_keys():
    with open(os.path.join(GOLDEN, "attend_hand.json")) as f:
        fx = json.load(f)
    lay = dict(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=2, block_q=1, block_k=2,
               q_len=1, q_valid=1, kv_prefix_len=0, kv_prefix_valid=0, kv_len=2,
               kv_suffix_valid=2, scale=1.0)
    q = synth.to_bf16_bits(np.array(fx["q"], float)).reshape(1, 1, 1, 2)
    k = synth.to_bf16_bits(np.array(fx["k"], float)).reshape(1, 2, 1, 2)
    v = synth.to_bf16_bits(np.array(fx["v"], float)).reshape(1, 2, 1, 2)
    idx, cnt = oracle.identity_selection(lay)
    o, lse = oracle.attend(lay, q, k, v, idx, cnt)
    assert np.abs(o[0, 0, 0] - np.array(fx["o"])).max() < 1e-15
    assert abs(lse[0, 0, 0] - fx["lse"]) < 1e-15


@pytest.mark.parametrize("fill", [float("nan"), 1.0e4])
def test_padding_invariance_and_unpadded_equivalence(fill):
    base = synth.make_case(hq=2, hkv=1, d=64, prefix=100, gen=300, cfg=29)
    dirty = synth.make_case(hq=2, hkv=1, d=64, prefix=100, gen=300, cfg=29, pad_fill=fill)
    idx, cnt = oracle.identity_selection(base.layout)
    o1, l1 = oracle.attend(base.layout, base.q, base.k, base.v, idx, cnt)
    o2, l2 = oracle.attend(dirty.layout, dirty.q, dirty.k, dirty.v, idx, cnt)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # dense over the padded layout == plain softmax attention over the
    # unpadded concatenation (torch SDPA without any mask)
    lay = base.layout
    keys = np.concatenate([np.arange(100), 128 + np.arange(300)])
    q = torch.from_numpy(_f64(base.q[0, :300])).permute(1, 0, 2)
    k = torch.from_numpy(_f64(base.k[0, keys])).permute(1, 0, 2).repeat_interleave(2, 0)
    v = torch.from_numpy(_f64(base.v[0, keys])).permute(1, 0, 2).repeat_interleave(2, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=float(np.float32(0.125)))
    assert np.abs(o1[0, :300] - ref.permute(1, 0, 2).numpy()).max() < 1e-12


@pytest.mark.parametrize("fill", [None, float("nan")])
def test_attend_rows_matches_attend(fill):
    case = synth.make_case(hq=4, hkv=2, d=64, prefix=50, gen=400, cfg=30, pad_fill=fill)
    lay = case.layout
    idx, cnt = oracle.select(lay, case.q, case.k, 4)
    o, lse = oracle.attend(lay, case.q, case.k, case.v, idx, cnt)
    rows = synth.sample_rows(case, 12)
    rows[..., -1] = lay["q_len"] - 1  # a padded query row
    orow, lrow = oracle.attend_rows(lay, case.q, case.k, case.v, idx, cnt, rows)
    assert lay["q_valid"] < lay["q_len"]
    for h in range(4):
        for r in range(12):
            t = rows[0, h, r]
            assert np.abs(orow[0, h, r] - o[0, t, h]).max() < 1e-13
            assert lrow[0, h, r] == lse[0, h, t] or abs(lrow[0, h, r] - lse[0, h, t]) < 1e-13
    assert (orow[0, :, -1] == 0).all() and np.isneginf(lrow[0, :, -1]).all()


def test_scale_default_is_inverse_sqrt_head_dim():
    case = synth.make_case(hq=2, hkv=1, d=64, prefix=0, gen=128, cfg=31)
    lay0 = dict(case.layout, scale=0.0)
    lay1 = dict(case.layout, scale=1 / math.sqrt(64))
    idx, cnt = oracle.identity_selection(case.layout)
    a, _ = oracle.attend(lay0, case.q, case.k, case.v, idx, cnt)
    b, _ = oracle.attend(lay1, case.q, case.k, case.v, idx, cnt)
    assert np.array_equal(a, b)
