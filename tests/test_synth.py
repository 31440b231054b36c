"""Seeded generator: deterministic bytes, layout, padding."""
import hashlib

import numpy as np

import synth


def _digest(case):
    h = hashlib.sha256()
    for a in (case.q, case.k, case.v):
        h.update(a.tobytes())
    return h.hexdigest()


def test_deterministic():
    a = synth.make_config("tiny")
    b = synth.make_config("tiny")
    assert _digest(a) == _digest(b)
    c = synth.make_case(gen=448, dist="normal", cfg=9)
    assert _digest(c) != _digest(a)


def test_tiny_layout():
    c = synth.make_config("tiny")
    lay = c.layout
    assert (lay["q_len"], lay["q_valid"], lay["kv_prefix_len"], lay["kv_len"]) == (448, 448, 64, 512)
    assert c.q.shape == (1, 448, 2, 64) and c.k.shape == (1, 512, 1, 64)
    assert lay["scale"] == 0.125


def test_padding_layout_and_zero_fill():
    c = synth.make_case(prefix=100, gen=200, bq=64, bk=64, hq=2, hkv=1, d=64)
    lay = c.layout
    assert lay["kv_prefix_len"] == 128 and lay["q_len"] == 256 and lay["kv_len"] == 128 + 256
    assert not c.q[:, 200:].any()
    assert not c.k[:, 100:128].any() and not c.k[:, 128 + 200:].any()
    assert c.k[:, :100].any() and c.k[:, 128:328].any()


def test_bf16_rounding_is_rne():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38])
    bits = synth.to_bf16_bits(vals)
    back = synth.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: even is 1 + 2^-6.
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2 ** -6 and back[3] == -2.5


def test_lowrank_component_norm():
    c = synth.make_case(gen=1560, frames=(1, 30, 52), dist="lowrank", hq=4, hkv=2, d=128, prefix=64,
                        cfg=3)
    n = synth.make_case(gen=1560, dist="normal", hq=4, hkv=2, d=128, prefix=64, cfg=3)
    # Same z draws: the difference is the structured part, of L2 norm 2 per token
    # (up to bf16 rounding of both).
    dq = synth.bf16_bits_to_f32(c.k[0, 64:64 + 1560]).astype(np.float64) - \
        synth.bf16_bits_to_f32(n.k[0, 64:64 + 1560]).astype(np.float64)
    norms = np.linalg.norm(dq, axis=-1)
    assert abs(norms.mean() - 2.0) < 0.05
    # prefix keys carry no structure
    assert np.array_equal(c.k[0, :64], n.k[0, :64])


def test_sample_rows_in_range():
    c = synth.make_config("tiny")
    rows = synth.sample_rows(c, 16)
    assert rows.shape == (1, 2, 16)
    assert rows.min() >= 0 and rows.max() < c.layout["q_valid"]
    assert (rows[:, :, 0] == 0).all() and (rows[:, :, 1] == c.layout["q_valid"] - 1).all()
