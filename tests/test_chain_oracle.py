"""Pins of the greedy chain oracle (oracle/chain.py): it equals the tree
oracle's k = 1 tree with every token a candidate (M = V), itself pinned by
brute-force enumeration; with W2 = 0 it is the per-depth argmax of the base
logits; relabelling the vocabulary relabels the chain."""
import numpy as np
import pytest

from oracle import chain, ref
from workloads import synth


def tiny(seed_shift=0):
    spec, w, req = synth.workload("tiny")
    return spec, w, req


def test_equals_k1_tree_with_all_candidates():
    spec, w, req = tiny()
    head = ref.make_head(w, False, False)
    base, hid, root = req["base"][0], req["hidden"][0].astype(np.float64), req["root"][0]
    toks, logits, margins = chain.greedy_chain(head, base, hid, root)
    t = ref.build_tree(head, base, hid, root, spec.V, 1, spec.D, 1.0, "topm")
    assert t.n_nodes == spec.D
    np.testing.assert_array_equal(toks, t.tokens[1:])
    np.testing.assert_array_equal(t.parents[1:], np.arange(spec.D))
    assert np.all(margins > 0)


def test_zero_w2_is_base_argmax():
    spec, w, req = tiny()
    w = dict(w)
    w["w2"] = np.zeros_like(w["w2"])
    head = ref.make_head(w, False, False)
    base = req["base"][0].copy()
    base[2, 17] = base[2].max()             # a tie at depth 3: the lower id wins
    toks, logits, _ = chain.greedy_chain(head, base, req["hidden"][0].astype(np.float64), req["root"][0])
    want = [int(np.flatnonzero(row == row.max())[0]) for row in base]
    np.testing.assert_array_equal(toks, want)
    np.testing.assert_array_equal(logits, base.max(axis=1).astype(np.float64))


def test_vocabulary_relabelling():
    spec, w, req = tiny()
    rng = np.random.default_rng(3)
    perm = rng.permutation(spec.V)          # new id of old token v is perm[v]
    inv = np.argsort(perm)
    w2 = dict(w)
    w2["emb"] = w["emb"][inv]
    w2["w2"] = w["w2"][:, inv]
    base = req["base"][0]
    hid, root = req["hidden"][0].astype(np.float64), req["root"][0]
    t0, l0, m0 = chain.greedy_chain(ref.make_head(w, False, False), base, hid, root)
    t1, l1, _ = chain.greedy_chain(ref.make_head(w2, False, False), base[:, inv], hid, root)
    assert np.all(m0 > 1e-9)                 # distinct maxima: the relabelling is exact
    np.testing.assert_array_equal(perm[t0], t1)
    np.testing.assert_allclose(l0, l1, rtol=0, atol=1e-12)


def test_fold_state_is_repeated_grucell():
    # library special case: torch.nn.GRUCell in float64 applied token by token
    import torch
    spec, w, req = tiny()
    head = ref.make_head(w, False, False)
    rng = np.random.default_rng(4)
    prev = rng.normal(0, 1, spec.ds)
    toks = rng.integers(0, spec.V, 5)
    got = chain.fold_state(head, prev, toks)
    cell = torch.nn.GRUCell(spec.e, spec.ds, bias=True).double()
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(np.asarray(w["w_ih"], np.float64)))
        cell.weight_hh.copy_(torch.from_numpy(np.asarray(w["w_hh"], np.float64)))
        cell.bias_ih.zero_()
        cell.bias_hh.zero_()
        h = torch.from_numpy(prev)[None]
        for t in toks:
            h = cell(torch.from_numpy(np.asarray(w["emb"][t], np.float64))[None], h)
    np.testing.assert_allclose(got, h[0].numpy(), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(chain.fold_state(head, prev, []), prev)
