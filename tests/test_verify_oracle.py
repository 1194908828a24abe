"""Pins of the tree-attention oracle (oracle/verify.py) against what the
definition fixes independently of it: the reflexive-transitive closure of the
parent relation (Warshall), the recursive form mask[i] = mask[parent(i)] + {i},
popcount = depth + 1, numpy's own bit packing, a hand-worked tree, and the
invariant checks on broken trees."""
import json
import os

import numpy as np
import pytest

from oracle import ref, verify
from workloads import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def random_tree(rng, cols, n):
    """A valid tree in the builder's layout: parents[i] < i, padding past n."""
    parents = np.full(cols, -1, np.int64)
    depths = np.full(cols, -1, np.int64)
    tokens = np.full(cols, -1, np.int64)
    depths[0] = 0
    for i in range(1, n + 1):
        parents[i] = rng.integers(0, i)
        depths[i] = depths[parents[i]] + 1
        tokens[i] = rng.integers(0, 1000)
    return parents, depths, tokens


def closure(parents, n):
    """Reflexive-transitive closure of 'j is the parent of i' on nodes 0..n,
    by Warshall's algorithm."""
    R = np.eye(n + 1, dtype=bool)
    for i in range(1, n + 1):
        R[i, parents[i]] = True
    for k in range(n + 1):
        R = R | (R[:, [k]] & R[[k], :])
    return R


@pytest.mark.parametrize("seed,cols,n", [(0, 9, 8), (1, 33, 32), (2, 65, 40), (3, 1, 0), (4, 129, 128)])
def test_mask_is_the_ancestor_closure(seed, cols, n):
    rng = np.random.default_rng(seed)
    parents, depths, tokens = random_tree(rng, cols, n)
    mask, pos, flat, bad = verify.tree_attention_inputs(parents, depths, tokens, n, prefix_len=17,
                                                        anchor=5)
    assert not bad
    np.testing.assert_array_equal(mask[:n + 1, :n + 1], closure(parents, n))
    assert not mask[n + 1:].any() and not mask[:, n + 1:].any()
    # recursive form and popcounts
    for i in range(1, n + 1):
        e = np.zeros(cols, bool)
        e[i] = True
        np.testing.assert_array_equal(mask[i], mask[parents[i]] | e)
    np.testing.assert_array_equal(mask[:n + 1].sum(1), depths[:n + 1] + 1)
    np.testing.assert_array_equal(pos[:n + 1], 17 + depths[:n + 1])
    assert np.all(pos[n + 1:] == -1) and np.all(flat[n + 1:] == -1)
    assert flat[0] == 5
    np.testing.assert_array_equal(flat[1:n + 1], tokens[1:n + 1])


def test_pack_matches_numpy_packbits():
    rng = np.random.default_rng(7)
    m = rng.random((5, 70)) < 0.5
    words = verify.pack_mask(m)
    pad = np.zeros((5, 96), bool)
    pad[:, :70] = m
    want = np.packbits(pad, axis=1, bitorder="little").view("<u4")
    np.testing.assert_array_equal(words, want)


def test_hand_worked_tree():
    # root 0 -> 1, 2; 1 -> 3; 3 -> 4; 2 -> 5 (written out by hand)
    g = json.load(open(os.path.join(GOLDEN, "tree_attention_hand.json")))
    mask, pos, flat, bad = verify.tree_attention_inputs(g["parents"], g["depths"], g["tokens"],
                                                        g["n_nodes"], g["prefix_len"], g["anchor"])
    assert not bad
    np.testing.assert_array_equal(verify.pack_mask(mask)[:, 0], np.array(g["mask_words"], np.uint32))
    np.testing.assert_array_equal(pos, g["positions"])
    np.testing.assert_array_equal(flat, g["flat_tokens"])


def test_builder_trees_are_valid():
    # the oracle's own trees on the tiny workload pass the invariant checks,
    # and every mask row is the node's path as ref.path_of walks it
    spec, w, req = synth.workload("tiny")
    t = ref.build_all(spec, w, req)[0]
    cols = spec.N + 1
    par = np.full(cols, -1, np.int64)
    dep = np.full(cols, -1, np.int64)
    tok = np.full(cols, -1, np.int64)
    par[:t.n_nodes + 1] = t.parents
    dep[:t.n_nodes + 1] = t.depths
    tok[:t.n_nodes + 1] = t.tokens
    mask, pos, flat, bad = verify.tree_attention_inputs(par, dep, tok, t.n_nodes)
    assert not bad
    for i in range(1, t.n_nodes + 1):
        path = ref.path_of(t.tokens, t.parents, i)
        assert mask[i].sum() == len(path) + 1       # the path's tokens plus the root


@pytest.mark.parametrize("case", ["parent_not_smaller", "depth_wrong", "n_too_big", "n_negative",
                                  "root_has_parent", "parent_below_minus_one"])
def test_broken_trees_are_bad(case):
    rng = np.random.default_rng(11)
    parents, depths, tokens = random_tree(rng, 17, 12)
    n = 12
    if case == "parent_not_smaller":
        parents[7] = 9
    elif case == "depth_wrong":
        depths[5] += 1
    elif case == "n_too_big":
        n = 17
    elif case == "n_negative":
        n = -3
    elif case == "root_has_parent":
        parents[0] = 0
    else:
        parents[4] = -2
    mask, pos, flat, bad = verify.tree_attention_inputs(parents, depths, tokens, n)
    assert bad
    assert mask.shape == (17, 17)
