"""Pins for the oracle's causal dense attention (bottom-right aligned over the
real tokens): torch's fp64 SDPA with ``is_causal=True`` on the CPU (a library
routine, top-left aligned) on the compacted real tokens, closed forms for
rows that see one key or every key, and padding invariance."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _real(case):
    """Compacted real tokens: q [B, n_q, Hq, D], k/v [B, n_k, Hkv, D] fp64."""
    lay = case.layout
    pl = lay["kv_prefix_len"]
    keys = np.r_[np.arange(lay["kv_prefix_valid"]), pl + np.arange(lay["kv_suffix_valid"])]
    return (_f64(case.q[:, :lay["q_valid"]]), _f64(case.k[:, keys]), _f64(case.v[:, keys]))


def _sdpa_causal(q, k, v, scale):
    """torch SDPA, fp64 CPU, is_causal (query i sees keys j <= i); GQA by
    repeating K/V heads. q [B, L, Hq, D], k/v [B, L, Hkv, D] with equal L."""
    hq, hkv = q.shape[2], k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def _scale(case):
    return float(np.float32(case.layout["scale"]))


CASES = [
    # (name, make_case kwargs): prefix = 0 and the queries are the stream itself
    ("square_gqa", dict(cfg=31, hq=4, hkv=2, d=64, bq=64, bk=64, prefix=0, gen=300)),
    ("square_mha_128", dict(cfg=32, hq=2, hkv=2, d=128, bq=128, bk=128, prefix=0, gen=333)),
    ("square_mqa_mixed", dict(cfg=33, hq=3, hkv=1, d=64, bq=128, bk=64, prefix=0, gen=200)),
]


@pytest.mark.parametrize("name,kw", CASES)
@pytest.mark.parametrize("fill", [None, float("nan")])
def test_square_equals_sdpa_causal(name, kw, fill):
    """A stream attending to itself: the usual causal mask, padding invisible."""
    case = synth.make_case(name, pad_fill=fill, **kw)
    lay = case.layout
    o, lse = oracle.dense_causal(lay, case.q, case.k, case.v)
    q, k, v = _real(case)
    ref = _sdpa_causal(q, k, v, _scale(case))
    n = lay["q_valid"]
    assert np.abs(o[:, :n] - ref).max() < 1e-12
    assert (o[:, n:] == 0).all() and np.isneginf(lse[:, :, n:]).all()
    # row 0 sees key 0 only: o = v_0 exactly, lse = scale q_0 . k_0
    grp = lay["num_q_heads"] // lay["num_kv_heads"]
    for h in range(lay["num_q_heads"]):
        assert np.array_equal(o[0, 0, h], v[0, 0, h // grp])
        assert math.isclose(lse[0, h, 0], _scale(case) * float(q[0, 0, h] @ k[0, 0, h // grp]),
                            rel_tol=1e-13, abs_tol=1e-13)


@pytest.mark.parametrize("fill", [None, float("nan")])
def test_bottom_right_with_prefix_is_tail_of_square(fill):
    """Generation rows over cat(prefix, gen): with n_k = P + G real keys and
    G real rows, row t sees every prefix key and generation keys <= t, i.e.
    the last G rows of a causal square over the concatenated real sequence."""
    case = synth.make_case("br", cfg=34, hq=4, hkv=1, d=64, bq=64, bk=64, prefix=100, gen=250,
                           pad_fill=fill)
    lay = case.layout
    o, lse = oracle.dense_causal(lay, case.q, case.k, case.v)
    q, k, v = _real(case)
    n_k, g = k.shape[1], q.shape[1]
    rng = np.random.default_rng(7)
    head = rng.standard_normal((1, n_k - g, q.shape[2], q.shape[3]))   # rows whose output is unused
    ref = _sdpa_causal(np.concatenate([head, q], axis=1), k, v, _scale(case))[:, n_k - g:]
    assert np.abs(o[:, :g] - ref).max() < 1e-12
    # the last real row sees every real key: the non-causal dense oracle's row
    od, lsed = oracle.dense(lay, case.q, case.k, case.v)
    assert np.abs(o[:, g - 1] - od[:, g - 1]).max() < 1e-12
    assert np.abs(lse[:, :, g - 1] - lsed[:, :, g - 1]).max() < 1e-12


def test_more_queries_than_keys():
    """n_q > n_k: the first n_q - n_k rows see no key (0, lse -inf); row t
    >= n_q - n_k is top-left causal row t - (n_q - n_k) of the square over
    the last n_k queries."""
    base = synth.make_case("wide", cfg=35, hq=2, hkv=1, d=64, bq=64, bk=64, prefix=0, gen=200)
    lay = dict(base.layout)
    kv_real = 150
    lay["kv_suffix_valid"] = kv_real               # keys 150.. of the segment become padding
    o, lse = oracle.dense_causal(lay, base.q, base.k, base.v)
    n_q = lay["q_valid"]
    shift = n_q - kv_real
    assert (o[:, :shift] == 0).all() and np.isneginf(lse[:, :, :shift]).all()
    q = _f64(base.q[:, shift:n_q])
    k = _f64(base.k[:, :kv_real])
    v = _f64(base.v[:, :kv_real])
    ref = _sdpa_causal(q, k, v, float(np.float32(lay["scale"])))
    assert np.abs(o[:, shift:n_q] - ref).max() < 1e-12


def test_key_ranks():
    lay = synth.make_layout(1, 1, 1, 64, 64, 64, prefix=70, gen=100)
    r = oracle.key_ranks(lay)
    assert r.shape == (lay["kv_len"],)
    assert np.array_equal(r[:70], np.arange(70)) and (r[70:128] == -1).all()
    assert np.array_equal(r[128:228], 70 + np.arange(100)) and (r[228:] == -1).all()


def test_alignment_matters():
    """With a prefix the two alignments differ by far more than the pins'
    tolerance: top-left alignment (row t sees keys <= t) is not what the
    oracle computes."""
    case = synth.make_case("br", cfg=34, hq=4, hkv=1, d=64, bq=64, bk=64, prefix=100, gen=250)
    lay = case.layout
    q, k, v = _real(case)
    n_k, g = k.shape[1], q.shape[1]
    wrong = _sdpa_causal(q, k[:, :g], v[:, :g], _scale(case))     # row t sees keys <= t only
    o, _ = oracle.dense_causal(lay, case.q, case.k, case.v)
    assert np.abs(o[:, :g] - wrong).max() > 1e-3
