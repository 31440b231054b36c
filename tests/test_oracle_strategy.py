"""Pins for the oracle's step/layer strategy: the call counts of the pages'
recipes (tests/golden/strategy_recipes.json, each with its citation) and the
composition of a strategy call from the pinned dense and selected paths."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from conftest import GOLDEN


def _layers(spec):
    if not spec:
        return []
    a, b = spec.split("-")
    return list(range(int(a), int(b) + 1))


RECIPES = json.load(open(os.path.join(GOLDEN, "strategy_recipes.json")))["recipes"]


@pytest.mark.parametrize("r", RECIPES, ids=[r["name"] for r in RECIPES])
def test_recipe_call_counts(r):
    layers = _layers(r["sparse_layers"])
    n_sparse = sum(oracle.strategy.is_sparse(r["num_layers"], r["dense_steps"], layers, s, l)
                   for s in range(r["steps"]) for l in range(r["num_layers"]))
    total = r["steps"] * r["num_layers"]
    assert n_sparse == r["sparse_calls"]
    assert total - n_sparse == r["dense_calls"]


def test_switch_happens_at_dense_steps():
    layers = list(range(8, 36))
    st = oracle.strategy
    assert not any(st.is_sparse(36, 10, layers, 9, l) for l in range(36))
    assert [st.is_sparse(36, 10, layers, 10, l) for l in range(36)] == [l >= 8 for l in range(36)]
    with pytest.raises(ValueError):
        st.is_sparse(36, 10, layers, 0, 36)


def test_layer_forward_composes_the_pinned_paths():
    case = synth.make_config("tiny")
    lay = case.layout
    o_d, l_d, sp = oracle.strategy.layer_forward(lay, case.q, case.k, case.v, 4, 2, [1, 3], 50, 1, 1)
    assert not sp
    rd, rdl = oracle.dense(lay, case.q, case.k, case.v)
    assert np.array_equal(o_d, rd) and np.array_equal(l_d, rdl)
    o_s, l_s, sp = oracle.strategy.layer_forward(lay, case.q, case.k, case.v, 4, 2, [1, 3], 50, 2, 3)
    assert sp
    idx, cnt = oracle.select(lay, case.q, case.k, 4)
    ro, rl = oracle.attend(lay, case.q, case.k, case.v, idx, cnt)
    assert np.array_equal(o_s, ro) and np.array_equal(l_s, rl)
    assert np.abs(o_s - o_d).max() > 1e-3   # 4 of 8 blocks differs from dense
