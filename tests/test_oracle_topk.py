"""Pins for the oracle's exact top-k.

The pages fix: the best k = 2,048 tokens are kept and below 2,048 tokens every
token is kept ("GLM on an A100, in Vx", section "The model"); ties follow a
stable argsort of -scores ("How do we know it is right?").  numpy's stable
argsort is that library routine, so tiny inputs are checked against it
directly, plus the invariants any exact top-k has."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np_topk(s, k, order="index"):
    sel = np.argsort(-np.asarray(s, np.float64), kind="stable")[:k]
    return np.sort(sel) if order == "index" else sel


def test_golden_relu_tie(oracle_mod):
    g = json.load(open(os.path.join(GOLDEN, "relu_tie_two_heads.json")))
    s = np.array([g["scores"]])
    for k, expect in g["topk"].items():
        idx, cnt = oracle_mod.topk(s, [len(g["scores"])], int(k))
        assert idx[0].tolist() == expect and cnt[0] == len(expect)
    for k, expect in g["topk_score_order"].items():
        idx, _ = oracle_mod.topk(s, [len(g["scores"])], int(k), order="score")
        assert idx[0].tolist() == expect


@pytest.mark.parametrize("n", [1, 63, 64, 65, 2047, 2048])
def test_context_at_most_k_selects_everything(oracle_mod, n):
    rng = np.random.default_rng(n)
    s = rng.standard_normal((1, 2048))
    idx, cnt = oracle_mod.topk(s, [n], 2048)
    assert cnt[0] == n
    assert idx[0, :n].tolist() == list(range(n))
    assert np.all(idx[0, n:] == -1)


def test_brute_force_tiny_all_k(oracle_mod):
    rng = np.random.default_rng(1)
    for trial in range(60):
        n = int(rng.integers(1, 65))
        # few distinct values: many exact ties
        s = rng.integers(-3, 4, size=n).astype(np.float64) * rng.choice([1.0, 0.5])
        for k in range(1, n + 3):
            for order in ("index", "score"):
                idx, cnt = oracle_mod.topk(s[None], [n], k, order=order)
                ref = _np_topk(s, k, order)
                assert cnt[0] == min(k, n)
                assert idx[0, :cnt[0]].tolist() == ref.tolist()
                assert np.all(idx[0, cnt[0]:] == -1)


def test_special_values_follow_numpy(oracle_mod):
    s = np.array([0.0, -0.0, np.nan, np.inf, -np.inf, 1.0, -0.0, np.nan, 0.0, -1.0, np.inf])
    n = len(s)
    for k in range(1, n + 1):
        for order in ("index", "score"):
            idx, _ = oracle_mod.topk(s[None], [n], k, order=order)
            assert idx[0, :k].tolist() == _np_topk(s, k, order).tolist()
    # -0.0 ties with +0.0: lowest index first
    idx, _ = oracle_mod.topk(np.array([[-0.0, 0.0, -0.0]]), [3], 1)
    assert idx[0, 0] == 0
    # NaN ranks below every number, -inf included
    idx, _ = oracle_mod.topk(np.array([[np.nan, -np.inf, np.nan]]), [3], 2, order="score")
    assert idx[0].tolist() == [1, 0]


def test_all_equal_keeps_lowest_indices(oracle_mod):
    s = np.full((2, 5000), 3.25)
    idx, cnt = oracle_mod.topk(s, [5000, 300], 2048)
    assert idx[0].tolist() == list(range(2048))
    assert idx[1, :300].tolist() == list(range(300)) and cnt[1] == 300


def test_rows_and_lengths_are_independent(oracle_mod):
    rng = np.random.default_rng(2)
    s = rng.standard_normal((4, 300))
    lens = [300, 17, 0, 129]
    idx, cnt = oracle_mod.topk(s, lens, 32)
    for i, n in enumerate(lens):
        ref = _np_topk(s[i, :n], 32)
        assert cnt[i] == min(32, n)
        assert idx[i, :cnt[i]].tolist() == ref.tolist()


@settings(max_examples=200, deadline=None)
@given(st.lists(st.sampled_from([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0, np.inf, -np.inf, np.nan]),
                min_size=1, max_size=80),
       st.integers(min_value=1, max_value=90))
def test_invariants_property(oracle_mod, vals, k):
    s = np.array(vals, np.float64)
    n = len(s)
    idx, cnt = oracle_mod.topk(s[None], [n], k)
    kept = idx[0, :cnt[0]]
    assert cnt[0] == min(k, n)
    assert len(set(kept.tolist())) == len(kept)
    assert kept.tolist() == sorted(kept.tolist())          # ascending index order
    dropped = np.setdiff1d(np.arange(n), kept)
    key = np.where(np.isnan(s), -np.inf, s)                 # NaN below everything
    isn = np.isnan(s)
    if len(dropped) and len(kept):
        # every kept score >= every dropped score (NaN lowest)
        def rank_key(i):
            return (0 if isn[i] else 1, key[i])
        assert min(rank_key(i) for i in kept) >= max(rank_key(i) for i in dropped)
        # at the boundary value, kept indices come before dropped ones
        low = min(rank_key(i) for i in kept)
        eq_kept = [i for i in kept if rank_key(i) == low]
        eq_drop = [i for i in dropped if rank_key(i) == low]
        if eq_drop:
            assert max(eq_kept) < min(eq_drop)
