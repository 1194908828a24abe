"""Pins of the chain oracle (oracle/chain.py).

Greedy: it equals the tree oracle's k = 1 tree with every token a candidate
(M = V), itself pinned by brute-force enumeration; with W2 = 0 it is the
per-depth argmax of the base logits; relabelling the vocabulary relabels the
chain.

Sampled: the generator reproduces the published Philox4x32-10 known-answer
vectors; the uniforms are the stated exact values; the Gumbel variates have
the distribution's mean and variance; Gumbel-max draws follow the softmax of
the tempered logits (a chi-square test); the sampled chain is the greedy
chain on the noise-perturbed logits, and the greedy chain as T goes to 0."""
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


# ---- sampled chain ----------------------------------------------------------

def test_philox_known_answers():
    # known-answer vectors published with Philox4x32-10 (Random123, the
    # implementation accompanying Salmon et al., SC 2011): counter, key, output
    m = 0xFFFFFFFF
    cases = [((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
             ((m, m, m, m), (m, m), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
             ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
              (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1))]
    for ctr, key, want in cases:
        got = chain.philox4x32_10(np.array(ctr, np.uint64), np.array(key, np.uint64))
        assert [int(x) for x in got] == list(want)


def test_chain_words_layout():
    # token v takes word v mod 4 of counter (v // 4, d, b, 0) under the
    # key (seed low word, seed high word)
    seed, b, d = 0x0123456789ABCDEF, 5, 3
    words = chain.chain_words(seed, b, d, 11)
    key = np.array([0x89ABCDEF, 0x01234567], np.uint64)
    for v in range(11):
        ctr = np.array([v // 4, d, b, 0], np.uint64)
        assert int(words[v]) == int(chain.philox4x32_10(ctr, key)[v % 4])


def test_uniforms_are_exact_and_open():
    w = np.array([0, 1, 511, 512, 2 ** 31, 2 ** 32 - 1], np.uint64)
    u = chain.uniforms(w)
    assert np.all((u > 0) & (u < 1))
    k = u * 2.0 ** 24
    np.testing.assert_array_equal(k, np.round(k))
    assert np.all(k.astype(np.int64) % 2 == 1)                  # odd multiples of 2^-24
    np.testing.assert_array_equal(u.astype(np.float32).astype(np.float64), u)
    assert u[0] == u[2] == 2.0 ** -24 and u[3] == 3 * 2.0 ** -24 and u[-1] == 1 - 2.0 ** -24


def test_gumbel_moments():
    # standard Gumbel: mean = Euler-Mascheroni constant, variance = pi^2 / 6
    words = np.concatenate([chain.chain_words(99, b, 0, 4096) for b in range(50)])
    g = chain.gumbel(chain.uniforms(words))
    n = g.size
    assert abs(g.mean() - np.euler_gamma) < 5 * np.sqrt(np.pi ** 2 / 6 / n)
    assert abs(g.var() - np.pi ** 2 / 6) < 0.05


def test_gumbel_max_draws_follow_the_tempered_softmax():
    from scipy import stats
    z = np.array([1.0, 0.2, -0.5, 2.0, 0.0, 1.3])
    T = 0.7
    p = np.exp(z / T - (z / T).max())
    p /= p.sum()
    n = 20000
    counts = np.zeros(z.size)
    for b in range(n):
        g = chain.gumbel(chain.uniforms(chain.chain_words(2024, b, 1, z.size)))
        counts[int(np.argmax(z / T + g))] += 1
    chi2 = ((counts - n * p) ** 2 / (n * p)).sum()
    assert stats.chi2.sf(chi2, z.size - 1) > 1e-4, (counts, n * p)
    # a sign error in the noise would favour the smallest logits instead
    assert np.argmax(counts) == np.argmax(z)


def test_sampled_chain_is_greedy_on_perturbed_logits():
    spec, w, req = tiny()
    head = ref.make_head(w, False, False)
    base, hid, root = req["base"][0], req["hidden"][0].astype(np.float64), req["root"][0]
    T, seed, row = 0.8, 77, 3
    toks, logits, margins = chain.sampled_chain(head, base, hid, root, T, seed, row)
    noise = np.stack([chain.gumbel(chain.uniforms(chain.chain_words(seed, row, d, spec.V)))
                      for d in range(spec.D)])
    gt, gl, gm = chain.greedy_chain(head, base + T * noise, hid, root)
    assert np.all(margins > 1e-9) and np.all(gm > 1e-9)
    np.testing.assert_array_equal(toks, gt)
    np.testing.assert_allclose(logits, gl - T * noise[np.arange(spec.D), gt], rtol=0, atol=1e-9)
    # the draws differ from the greedy chain (with this seed)
    g0, _, _ = chain.greedy_chain(head, base, hid, root)
    assert not np.array_equal(toks, g0)


def test_sampled_chain_at_low_temperature_is_greedy():
    spec, w, req = tiny()
    head = ref.make_head(w, False, False)
    base, hid, root = req["base"][0], req["hidden"][0].astype(np.float64), req["root"][0]
    g0, l0, m0 = chain.greedy_chain(head, base, hid, root)
    assert m0.min() > 1e-3
    toks, logits, _ = chain.sampled_chain(head, base, hid, root, 1e-6, 5, 0)
    np.testing.assert_array_equal(toks, g0)
    np.testing.assert_array_equal(logits, l0)


def test_sampled_chain_depends_on_seed_and_row_only():
    spec, w, req = tiny()
    head = ref.make_head(w, False, False)
    base, hid, root = req["base"][0], req["hidden"][0].astype(np.float64), req["root"][0]
    a = chain.sampled_chain(head, base, hid, root, 1.0, 11, 0)[0]
    np.testing.assert_array_equal(a, chain.sampled_chain(head, base, hid, root, 1.0, 11, 0)[0])
    others = [chain.sampled_chain(head, base, hid, root, 1.0, 12, 0)[0],
              chain.sampled_chain(head, base, hid, root, 1.0, 11, 1)[0]]
    assert all(not np.array_equal(a, o) for o in others)
