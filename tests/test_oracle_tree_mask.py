"""Pins of the oracle's tree attention mask and position ids (no GPU).

Page: [ZH] "投机解码与 EAGLE：步骤、发展历史与三代差异" (caijizhuo.github.io),
section 3 ("草稿树与树形注意力掩码"): the draft tree is flattened into numbered
nodes and every node attends only to itself and its ancestors, not to its
siblings; the default EAGLE-1 tree has 25 nodes and depth 5.  Each pin below
checks the oracle against a definition it does not use: the causal mask of a
chain, reachability by boolean matrix powers, the recursive definition
row(n) = row(parent(n)) + {n}, and the creation level the dynamic-tree
generator records for every node.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth


def _bits(mask_row: np.ndarray, nn: int) -> np.ndarray:
    """Unpack one row of 64-bit words into nn booleans (bit j of word j//64)."""
    words = mask_row.astype(np.uint64)
    return np.array([(int(words[j // 64]) >> (j % 64)) & 1 for j in range(nn)], dtype=bool)


def _unpack(mask: np.ndarray, nn: int) -> np.ndarray:
    B = mask.shape[0]
    return np.stack([np.stack([_bits(mask[b, n], nn) for n in range(nn)]) for b in range(B)])


def _closure(parents) -> np.ndarray:
    """Ancestor-or-self relation by boolean matrix powers of the parent map."""
    nn = len(parents)
    step = np.zeros((nn, nn), dtype=np.int64)   # step[n, p] = 1 if p is n's parent
    for n in range(1, nn):
        step[n, parents[n]] = 1
    reach = np.eye(nn, dtype=np.int64)
    power = np.eye(nn, dtype=np.int64)
    for _ in range(nn):
        power = (power @ step > 0).astype(np.int64)
        reach |= power
    return reach.astype(bool)


@pytest.mark.parametrize("nn", [1, 2, 7, 64, 65, 130])
def test_chain_is_the_causal_mask(nn):
    """A chain (parent[n] = n - 1) sees exactly nodes 0..n: the lower-triangular
    causal mask, including rows spread over several 64-bit words."""
    parents = np.array([-1] + list(range(nn - 1)), np.int32)
    mask, pos = oracle.tree_mask(parents, np.array([5], np.int32), B=1)
    assert mask.shape == (1, nn, (nn + 63) // 64)
    assert np.array_equal(_unpack(mask, nn)[0], np.tril(np.ones((nn, nn), dtype=bool)))
    assert np.array_equal(pos[0], 5 + np.arange(nn))


def test_star_sees_root_and_self():
    nn = 12
    parents = np.array([-1] + [0] * (nn - 1), np.int32)
    mask, pos = oracle.tree_mask(parents, None, B=1)
    want = np.eye(nn, dtype=bool)
    want[:, 0] = True
    assert np.array_equal(_unpack(mask, nn)[0], want)
    assert pos[0].tolist() == [0] + [1] * (nn - 1)


@pytest.mark.parametrize("nn", [1, 2, 3, 4, 5, 6])
def test_every_small_tree_by_matrix_powers(nn):
    """Every valid parent array with nn <= 6 nodes (parent[n] in [0, n)):
    the mask equals reachability by matrix powers, and the position is the
    number of strict ancestors."""
    choices = [range(n) for n in range(1, nn)]
    arrays = [np.array([-1] + list(c), np.int32) for c in itertools.product(*choices)]
    P = np.stack(arrays)
    L0 = np.arange(len(arrays), dtype=np.int32) * 3
    mask, pos = oracle.tree_mask(P, L0)
    got = _unpack(mask, nn)
    for i, par in enumerate(arrays):
        reach = _closure(par)
        assert np.array_equal(got[i], reach), par
        assert np.array_equal(pos[i], L0[i] + reach.sum(axis=1) - 1), par


def test_eagle1_default_tree_recursive_definition():
    """The 25-node, depth-5 static tree: row(n) = row(parent(n)) + {n}, siblings
    never see each other, and the deepest nodes sit 5 levels below the root."""
    parents = np.array(synth.STATIC_TREE_PARENTS, np.int32)
    nn = len(parents)
    assert nn == 26
    mask, pos = oracle.tree_mask(parents, np.array([100, 7], np.int32), B=2)
    rows = _unpack(mask, nn)
    for b in range(2):
        assert rows[b, 0].tolist() == [True] + [False] * (nn - 1)
        for n in range(1, nn):
            want = rows[b, parents[n]].copy()
            want[n] = True
            assert np.array_equal(rows[b, n], want)
        for n in range(1, nn):
            for m in range(1, nn):
                if m != n and parents[m] == parents[n]:
                    assert not rows[b, n, m]
    assert pos[0].max() - 100 == 5 and pos[1].min() == 7


def test_positions_match_the_generators_levels():
    """Per-sequence dynamic trees (the dynamic-tree recipe, small V): position - L0 is
    the level the generator created each node at."""
    w = synth.WORKLOADS["tree_dynamic_b128_v152064"].with_sizes(V=512)
    inp = synth.dynamic_tree_inputs(w, seed=3, B=6)
    L0 = np.array([0, 1, 17, 400, 4095, 9], np.int32)
    mask, pos = oracle.tree_mask(inp["parents"].numpy(), L0)
    assert np.array_equal(pos - L0[:, None], inp["depth_of"].numpy())


def test_bad_parents_mark_only_their_sequence():
    good = [-1, 0, 0, 1]
    bad = [[0, 0, 0, 1],      # root not -1
           [-1, 0, 2, 1],     # parent not below the node
           [-1, 0, -1, 1],    # negative parent
           [-1, 0, 0, 4]]     # parent past the node
    P = np.array([good] + bad + [good], np.int32)
    mask, pos = oracle.tree_mask(P, None)
    for b in range(1, 5):
        assert (mask[b] == 0).all() and (pos[b] == -1).all()
    for b in (0, 5):
        assert pos[b].tolist() == [0, 1, 1, 2]
        assert [int(x) for x in mask[b, :, 0]] == [0b1, 0b11, 0b101, 0b1011]
