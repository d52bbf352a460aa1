"""Pins of the oracle's EAGLE-2 dynamic draft tree (no GPU).

Page: [ZH] "投机解码与 EAGLE：步骤、发展历史与三代差异" (caijizhuo.github.io):
section 4, "eagle_round" step 2 (each frontier node adds its top-k draft
tokens with score = parent score x p(token); the best nodes grow next) and
section 5 (EAGLE-2 allots nodes globally by that score and keeps a budget).
Each pin checks the oracle against something it does not compute itself:
the synthetic generator's independent torch construction, numpy argmax /
stable argsort, scipy's log-softmax, and structural facts of the recipe.
"""
import numpy as np
import pytest
from scipy.special import log_softmax

import oracle
import synth


def _rows(B, depth, topk, V, seed, scale=3.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, 1 + topk * (depth - 1), V)) * scale).astype(np.float32)


@pytest.mark.parametrize("V,seed", [(512, 3), (3000, 11)])
def test_matches_the_generators_construction(V, seed):
    """The dynamic-tree recipe (depth 6, top-10, budget 60) on fp32 rows at T = 1:
    the oracle's tree equals the one the input generator grows with torch
    (log_softmax in double, stable sorts)."""
    w = synth.WORKLOADS["tree_dynamic_b128_v152064"].with_sizes(V=V, dtype="f32", T=1.0)
    inp = synth.dynamic_tree_inputs(w, seed=seed, B=6)
    o = oracle.tree_build(inp["expanded_p"].numpy(), w.depth, w.topk, w.budget, w.T)
    assert np.array_equal(o["parents"], inp["parents"].numpy())
    assert np.array_equal(o["tokens"], inp["tokens"].numpy())
    assert np.array_equal(o["depth"], inp["depth_of"].numpy())


def test_top1_is_the_greedy_chain():
    depth, V = 5, 300
    rows = _rows(4, depth, 1, V, 1)
    o = oracle.tree_build(rows, depth, 1, depth, 1.0)
    for b in range(4):
        assert o["parents"][b].tolist() == [-1] + list(range(depth))
        assert o["tokens"][b, 1:].tolist() == [int(np.argmax(rows[b, l])) for l in range(depth)]
        assert o["depth"][b].tolist() == list(range(depth + 1))


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_depth1_is_the_roots_topk(T):
    k, V = 7, 400
    rows = _rows(3, 1, k, V, 2)
    o = oracle.tree_build(rows, 1, k, k, T)
    T32 = float(np.float32(T))
    for b in range(3):
        want = np.argsort(-rows[b, 0].astype(np.float64), kind="stable")[:k]
        assert o["tokens"][b, 1:].tolist() == want.tolist()
        assert (o["parents"][b, 1:] == 0).all() and (o["depth"][b, 1:] == 1).all()
        lp = log_softmax(rows[b, 0].astype(np.float64) / T32)
        assert np.allclose(o["score"][b, 1:], lp[want], rtol=0, atol=1e-12)


def test_level2_scores_are_path_sums():
    """A level-2 node's score is ln p_root(parent token) + ln p_row(token),
    the row being the one its parent was expanded with (its frontier rank)."""
    depth, k, V, B = 2, 4, 200, 5
    rows = _rows(B, depth, k, V, 4)
    o = oracle.tree_build(rows, depth, k, k + k * k, 1.0)
    for b in range(B):
        lp_root = log_softmax(rows[b, 0].astype(np.float64))
        root_top = np.argsort(-rows[b, 0].astype(np.float64), kind="stable")[:k]
        for node in range(1, k + k * k + 1):
            if o["depth"][b, node] != 2:
                continue
            ptok = o["tokens"][b, o["parents"][b, node]]
            pid = int(np.where(root_top == ptok)[0][0])          # candidate id of the parent
            rank = int(np.where(o["frontier"][b, 0] == pid)[0][0])
            lp = log_softmax(rows[b, 1 + rank].astype(np.float64))
            assert abs(o["score"][b, node] - (lp_root[ptok] + lp[o["tokens"][b, node]])) < 1e-12


def test_full_budget_keeps_every_candidate():
    depth, k, V = 4, 3, 100
    n = k + (depth - 1) * k * k
    o = oracle.tree_build(_rows(2, depth, k, V, 5), depth, k, n, 1.0)
    for b in range(2):
        counts = np.bincount(o["depth"][b], minlength=depth + 1)
        assert counts.tolist() == [1, k] + [k * k] * (depth - 1)


def test_structure_of_the_kept_tree():
    """Parents precede children, depth grows by one per edge, a child never
    outscores its parent, and within a level scores do not increase."""
    w = synth.WORKLOADS["tree_dynamic_b128_v152064"]
    rows = _rows(4, w.depth, w.topk, 2000, 6)
    o = oracle.tree_build(rows, w.depth, w.topk, w.budget, 0.7)
    for b in range(4):
        P, D, S = o["parents"][b], o["depth"][b], o["score"][b]
        for n in range(1, w.budget + 1):
            assert 0 <= P[n] < n and D[n] == D[P[n]] + 1 and S[n] <= S[P[n]]
            if D[n] == D[n - 1]:
                assert S[n] <= S[n - 1]
        assert (np.diff(D) >= 0).all()


def test_ties_go_to_the_lower_token():
    """A row of equal logits: its top-k are tokens 0..k-1, in order."""
    rows = np.zeros((1, 1, 50), np.float32)
    o = oracle.tree_build(rows, 1, 5, 5, 1.0)
    assert o["tokens"][0, 1:].tolist() == [0, 1, 2, 3, 4]


def test_bad_row_fails_only_its_sequence():
    depth, k, V = 3, 2, 64
    rows = _rows(3, depth, k, V, 7)
    rows[1, 2, 10] = np.nan
    o = oracle.tree_build(rows, depth, k, 5, 1.0)
    assert (o["parents"][1] == -1).all() and (o["tokens"][1] == -1).all()
    for b in (0, 2):
        assert o["parents"][b, 0] == -1 and (o["parents"][b, 1:] >= 0).all()
