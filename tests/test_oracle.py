"""Pins of the CPU oracle against facts it does not compute itself.

Each test checks the oracle against a closed form, a library routine that
implements the same definition independently, brute force on tiny inputs,
an invariant stated by the pages, or a hand-worked fixture in tests/golden/.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import certify, ref
from workloads import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers


def _head_from(spec, w):
    return ref.make_head(w, spec.wdtype == "bf16", spec.act_bf16)


def _zero_weights(V, D, h, ds, r):
    return {
        "emb": np.zeros((V, h), np.float32),
        "w_ih": np.zeros((3 * ds, h), np.float32),
        "w_hh": np.zeros((3 * ds, ds), np.float32),
        "w1": np.zeros((h + ds, r), np.float32),
        "w2": np.zeros((r, V), np.float32),
        "b_ih": None, "b_hh": None, "w_lm": None,
    }


def _tree_paths(t):
    return [tuple(ref.path_of(t.tokens, t.parents, i)) for i in range(1, t.n_nodes + 1)]


def _small_case(seed, V=5, D=3, M=None, k=None, N=10, T=1.0, norm="topm", wdtype="f32",
                biases=True, root_std=0.5):
    spec = synth.small(f"s{seed}", V=V, D=D, M=M, k=k, N=N, T=T, group=1000 + seed,
                       norm=norm, wdtype=wdtype, biases=biases, root_std=root_std)
    spec, w, req = synth.workload(spec)
    return spec, w, req


# ----------------------------------------------------------------------------
# elementary pieces


def test_round_bf16_matches_torch_and_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    assert ref.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert ref.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert ref.round_bf16(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == -(1 + 2.0 ** -6)
    x = np.random.default_rng(0).standard_normal(20000) * 3
    lib = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ref.round_bf16(x), lib)


def test_bf16_values_widen_exactly():
    x = np.random.default_rng(1).standard_normal(5000).astype(np.float32)
    bits = synth.bf16_bits(x)
    lib = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ref.bf16_values(bits), lib)


def test_logsumexp_matches_scipy():
    rng = np.random.default_rng(2)
    for n in (1, 2, 7, 1000):
        x = rng.standard_normal(n) * 10
        assert abs(ref.logsumexp(x) - scipy.special.logsumexp(x)) < 1e-12
    assert ref.logsumexp(np.array([])) == -math.inf
    assert ref.logsumexp(np.array([-math.inf, -math.inf])) == -math.inf
    assert ref.logsumexp(np.array([-math.inf, 0.0])) == 0.0


def test_gru_matches_torch_grucell():
    rng = np.random.default_rng(3)
    e, ds = 7, 5
    w = {"emb": rng.standard_normal((4, e)).astype(np.float32),
         "w_ih": rng.standard_normal((3 * ds, e)).astype(np.float32),
         "w_hh": rng.standard_normal((3 * ds, ds)).astype(np.float32),
         "b_ih": rng.standard_normal(3 * ds).astype(np.float32),
         "b_hh": rng.standard_normal(3 * ds).astype(np.float32),
         "w1": np.zeros((e + ds, 3), np.float32), "w2": np.zeros((3, 4), np.float32)}
    head = ref.make_head(w, bf16=False, act_bf16=False)
    cell = torch.nn.GRUCell(e, ds, dtype=torch.float64)
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(w["w_ih"].astype(np.float64)))
        cell.weight_hh.copy_(torch.from_numpy(w["w_hh"].astype(np.float64)))
        cell.bias_ih.copy_(torch.from_numpy(w["b_ih"].astype(np.float64)))
        cell.bias_hh.copy_(torch.from_numpy(w["b_hh"].astype(np.float64)))
    for _ in range(5):
        s = rng.standard_normal(ds)
        x = rng.standard_normal(e)
        want = cell(torch.from_numpy(x)[None], torch.from_numpy(s)[None])[0].detach().numpy()
        np.testing.assert_allclose(ref.gru_step(head, s, x), want, rtol=0, atol=1e-13)


def test_gru_closed_forms():
    ds, e = 3, 2
    w = _zero_weights(4, 1, e, ds, 2)
    s = np.array([0.3, -1.2, 2.0])
    x = np.array([0.7, -0.4])
    # all-zero weights: r = z = 1/2, n = tanh(0) = 0, so S' = S / 2
    head = ref.make_head(w, False, False)
    np.testing.assert_allclose(ref.gru_step(head, s, x), 0.5 * s, atol=1e-15)
    # a large positive update-gate bias keeps the state
    w2 = dict(w, b_ih=np.r_[np.zeros(ds), np.full(ds, 60.0), np.zeros(ds)].astype(np.float32))
    np.testing.assert_allclose(ref.gru_step(ref.make_head(w2, False, False), s, x), s,
                               atol=1e-12)
    # a large negative update-gate bias with W_hn = 0 gives tanh(W_in x + b_in)
    w_in = np.array([[0.5, 1.0], [-2.0, 0.25], [0.0, 3.0]], np.float32)
    w3 = dict(w, w_ih=np.r_[np.zeros((2 * ds, e)), w_in].astype(np.float32),
              b_ih=np.r_[np.zeros(ds), np.full(ds, -60.0), [0.1, 0.2, -0.3]].astype(np.float32))
    want = np.tanh(w_in.astype(np.float64) @ x + np.array([0.1, 0.2, -0.3], np.float32))
    np.testing.assert_allclose(ref.gru_step(ref.make_head(w3, False, False), s, x), want,
                               atol=1e-12)


def test_gru_one_unit_worked_example():
    # x = 1, s = 0.5; reset pre-activation 0 -> r = 1/2; update pre-activation
    # ln 3 -> z = 3/4; new gate tanh(0.3 + r * 0.8 * 0.5) = tanh(0.5).
    w = {"emb": np.zeros((1, 1), np.float32),
         "w_ih": np.array([[0.0], [math.log(3.0)], [0.3]]),
         "w_hh": np.array([[0.0], [0.0], [0.8]]),
         "b_ih": None, "b_hh": None,
         "w1": np.zeros((2, 1)), "w2": np.zeros((1, 1))}
    head = ref.make_head(w, False, False)
    got = ref.gru_step(head, np.array([0.5]), np.array([1.0]))[0]
    assert abs(got - (0.25 * math.tanh(0.5) + 0.75 * 0.5)) < 1e-15


def test_bf16_state_rounding_only_in_matrix_products():
    # w_ih = 0, r/z rows of w_hh = 0 (r = z = 1/2), n rows of w_hh = I:
    # S' = tanh(bf16(S) / 2) / 2 + S / 2; S = 1 + 2^-10 has bf16(S) = 1.
    ds = 2
    w = _zero_weights(3, 1, 2, ds, 2)
    w["w_hh"] = np.r_[np.zeros((2 * ds, ds)), np.eye(ds)].astype(np.float32)
    s = np.array([1 + 2.0 ** -10, -3.0])
    head = ref.make_head(w, bf16=False, act_bf16=True)
    want = 0.5 * np.tanh(0.5 * np.array([1.0, -3.0])) + 0.5 * s
    np.testing.assert_allclose(ref.gru_step(head, s, np.zeros(2)), want, atol=1e-15)
    head_full = ref.make_head(w, bf16=False, act_bf16=False)
    want_full = 0.5 * np.tanh(0.5 * s) + 0.5 * s
    np.testing.assert_allclose(ref.gru_step(head_full, s, np.zeros(2)), want_full, atol=1e-15)


def test_correction_matches_full_vocab_torch_and_zero_cases():
    rng = np.random.default_rng(4)
    V, h, ds, r = 11, 6, 4, 5
    w = {"emb": rng.standard_normal((V, 3)).astype(np.float32),
         "w_ih": np.zeros((3 * ds, 3), np.float32), "w_hh": np.zeros((3 * ds, ds), np.float32),
         "b_ih": None, "b_hh": None,
         "w1": rng.standard_normal((h + ds, r)).astype(np.float32),
         "w2": rng.standard_normal((r, V)).astype(np.float32)}
    head = ref.make_head(w, False, False)
    hd, s = rng.standard_normal(h), rng.standard_normal(ds)
    cand = np.array([7, 2, 9])
    # full-vocabulary correction, then the candidate columns
    x = torch.cat([torch.from_numpy(hd), torch.from_numpy(s)])
    full = torch.from_numpy(w["w2"].astype(np.float64)).T @ torch.nn.functional.silu(
        x @ torch.from_numpy(w["w1"].astype(np.float64)))
    np.testing.assert_allclose(ref.correction(head, hd, s, cand), full.numpy()[cand],
                               atol=1e-13)
    # the H half of W1 multiplies H_d, the S half multiplies S
    w_h = dict(w, w1=np.r_[w["w1"][:h], np.zeros((ds, r), np.float32)])
    a = np.asarray(hd @ w["w1"][:h].astype(np.float64))
    np.testing.assert_allclose(ref.correction(ref.make_head(w_h, False, False), hd, s, cand),
                               w["w2"][:, cand].T.astype(np.float64) @ (a / (1 + np.exp(-a))),
                               atol=1e-13)
    # W2 = 0 or W1 = 0 gives no correction (SiLU(0) = 0)
    for zw in (dict(w, w2=np.zeros_like(w["w2"])), dict(w, w1=np.zeros_like(w["w1"]))):
        assert np.all(ref.correction(ref.make_head(zw, False, False), hd, s, cand) == 0)


def test_candidates_order_ties_zero_and_inf():
    row = np.array([1.0, 3.0, -0.0, 3.0, 0.0, -np.inf, 2.0])
    d = ref.candidates(row, 6, 1.0)
    # 3.0 twice (ids 1, 3), 2.0, 1.0, then the signed zeros tie (ids 2, 4)
    assert d.cand.tolist() == [1, 3, 6, 0, 2, 4]
    assert d.margin == math.inf                  # next is -inf
    d = ref.candidates(row, 5, 1.0)
    assert d.cand.tolist() == [1, 3, 6, 0, 2] and d.margin == 0.0
    rng = np.random.default_rng(5)
    x = rng.standard_normal(1000).astype(np.float32)
    d = ref.candidates(x, 37, 1.0)
    want = torch.topk(torch.from_numpy(x), 37).indices.numpy()
    assert d.cand.tolist() == want.tolist()
    # -inf sorts last
    d = ref.candidates(np.array([-np.inf, -np.inf, 0.5]), 3, 1.0)
    assert d.cand.tolist() == [2, 0, 1]


def test_candidate_lse_and_tail():
    rng = np.random.default_rng(6)
    x = rng.standard_normal(300) * 2
    for T in (1.0, 0.5):
        d = ref.candidates(x, 17, T)
        assert abs(d.lse - scipy.special.logsumexp(x / T)) < 1e-12
        rest = np.setdiff1d(np.arange(300), d.cand)
        assert abs(d.tail - scipy.special.logsumexp(x[rest] / T)) < 1e-12


# ----------------------------------------------------------------------------
# hand-worked trees


def _fixture_case(fx):
    V, D = fx["V"], fx["D"]
    w = _zero_weights(V, D, 2, 2, 2)
    if "probs" in fx:
        base = np.log(np.array(fx["probs"]))
    else:
        base = np.array(fx["logits"], np.float64)
    head = ref.make_head(w, False, False)
    t = ref.build_tree(head, base, np.zeros((D, 2)), np.zeros(2), fx["M"], fx["k"], fx["N"],
                       fx["T"])
    return t


def test_golden_hand_tree_distinct_scores():
    fx = json.load(open(os.path.join(GOLDEN, "hand_tree_distinct.json")))
    t = _fixture_case(fx)
    ex = fx["expected"]
    assert t.tokens == ex["tokens"]
    assert t.parents == ex["parents"]
    assert t.depths == ex["depths"]
    np.testing.assert_allclose(np.exp(t.scores), ex["path_probs"], atol=1e-15)


def test_golden_hand_tree_ties():
    fx = json.load(open(os.path.join(GOLDEN, "hand_tree_ties.json")))
    t = _fixture_case(fx)
    ex = fx["expected"]
    assert t.tokens == ex["tokens"]
    assert t.parents == ex["parents"]
    assert t.depths == ex["depths"]
    assert t.scores == [c * math.log(2.0) for c in ex["scores_in_ln2"]]


# ----------------------------------------------------------------------------
# brute force


def _enumerate(head, deps, hidden, root, D, k, T, norm):
    """Every node of the k-restricted tree with its path score (no heap).

    Children of a node: the k best candidates of the next depth by
    (corrected logit desc, token asc), with finite log-prob.
    """
    out = []

    def rec(path, s, score):
        d = len(path) + 1
        if d > D:
            return
        dep = deps[d - 1]
        ex = ref.expand_scores(head, dep, hidden[d - 1], s, len(dep.cand), T, norm)
        order = sorted(range(len(dep.cand)), key=lambda m: (-ex.z[m], int(dep.cand[m])))
        for m in order[:k]:
            if not np.isfinite(ex.logp[m]):
                continue
            tok = int(dep.cand[m])
            sc = score + float(ex.logp[m])
            out.append((path + (tok,), sc))
            rec(path + (tok,), ref.gru_step(head, s, head.emb(tok)), sc)

    rec((), np.asarray(root, np.float64), 0.0)
    return out


def _best_first_prefix(nodes, N):
    keys = [(-sc, len(p), p[-1]) for p, sc in nodes]
    assert len(set(keys)) == len(keys), "exact tie: brute force cannot rank parents"
    return sorted(nodes, key=lambda t: (-t[1], len(t[0]), t[0][-1]))[:N]


@pytest.mark.parametrize("seed,V,D,M,k,N,T,norm", [
    (0, 4, 3, None, None, 20, 1.0, "topm"),
    (1, 5, 3, None, None, 40, 1.0, "topm"),
    (2, 6, 3, None, None, 60, 0.5, "topm"),
    (3, 3, 4, None, None, 50, 1.0, "fullv"),
    (4, 5, 3, None, None, 155, 1.0, "topm"),     # the whole tree (5 + 25 + 125)
])
def test_brute_force_unlimited_k(seed, V, D, M, k, N, T, norm):
    spec, w, req = _small_case(seed, V=V, D=D, M=M, k=k, N=N, T=T, norm=norm)
    head = _head_from(spec, w)
    hid = req["hidden"][0].astype(np.float64)
    t = ref.build_tree(head, req["base"][0], hid, req["root"][0], spec.M, spec.k, N, T, norm)
    # score_path on every path of the full tree, independently of the heap
    deps = t.depths_info
    allp = []
    for d in range(1, D + 1):
        for path in itertools.product(range(V), repeat=d):
            sc, _ = ref.score_path(head, deps, hid, req["root"][0], list(path), T, norm)
            allp.append((tuple(path), sc))
    want = _best_first_prefix(allp, N)
    assert _tree_paths(t) == [p for p, _ in want]
    np.testing.assert_allclose(t.scores[1:], [s for _, s in want], atol=1e-12)


@pytest.mark.parametrize("seed,V,D,M,k,N,T,norm", [
    (10, 6, 4, 6, 2, 25, 1.0, "topm"),
    (11, 6, 4, 4, 3, 40, 1.0, "fullv"),
    (12, 5, 3, 3, 1, 10, 1.0, "topm"),
    (13, 6, 4, 5, 2, 31, 0.5, "fullv"),
])
def test_brute_force_finite_k(seed, V, D, M, k, N, T, norm):
    spec, w, req = _small_case(seed, V=V, D=D, M=M, k=k, N=N, T=T, norm=norm)
    head = _head_from(spec, w)
    hid = req["hidden"][0].astype(np.float64)
    t = ref.build_tree(head, req["base"][0], hid, req["root"][0], M, k, N, T, norm)
    nodes = _enumerate(head, t.depths_info, hid, req["root"][0], D, k, T, norm)
    want = _best_first_prefix(nodes, N)
    assert _tree_paths(t) == [p for p, _ in want]
    np.testing.assert_allclose(t.scores[1:], [s for _, s in want], atol=1e-12)


def test_brute_force_bf16_weights():
    spec, w, req = _small_case(20, V=6, D=3, M=5, k=3, N=20, wdtype="bf16")
    assert spec.act_bf16
    head = _head_from(spec, w)
    hid = ref.bf16_values(req["hidden"][0])
    t = ref.build_tree(head, req["base"][0], hid, req["root"][0], 5, 3, 20, 1.0)
    nodes = _enumerate(head, t.depths_info, hid, req["root"][0], 3, 3, 1.0, "topm")
    assert _tree_paths(t) == [p for p, _ in _best_first_prefix(nodes, 20)]


# ----------------------------------------------------------------------------
# invariants and special cases


def _product_tree(base, M, k, N, T, norm, dl=None):
    """Best-first prefix of the factorised (position-only) tree, by enumeration.

    depth d's children are the k best of its M candidates by
    (base + dl_d) desc, token asc; their log-prob is the depth's log-softmax
    over the candidates (topm) or candidates plus base tail (fullv).
    """
    D, V = base.shape
    per = []
    for d in range(D):
        row = base[d].astype(np.float64)
        ids = sorted(range(V), key=lambda v: (-row[v], v))[:M]
        rest = [v for v in range(V) if v not in ids]
        z = (row[ids] + (0 if dl is None else dl[d])) / T
        norm_terms = list(z) + ([scipy.special.logsumexp(row[rest] / T)]
                                if norm == "fullv" and rest else [])
        lz = scipy.special.logsumexp(norm_terms)
        best = sorted(range(M), key=lambda m: (-z[m], ids[m]))[:k]
        per.append([(ids[m], z[m] - lz) for m in best])
    nodes = []
    for d in range(1, D + 1):
        for combo in itertools.product(*per[:d]):
            nodes.append((tuple(t for t, _ in combo), float(sum(lp for _, lp in combo))))
    return _best_first_prefix(nodes, N)


@pytest.mark.parametrize("norm", ["topm", "fullv"])
def test_w2_zero_gives_factorised_tree(norm):
    spec, w, req = _small_case(30, V=7, D=4, M=5, k=3, N=30, norm=norm)
    w = dict(w, w2=np.zeros_like(w["w2"]))
    head = _head_from(spec, w)
    t = ref.build_tree(head, req["base"][0], req["hidden"][0].astype(np.float64),
                       req["root"][0], 5, 3, 30, 1.0, norm)
    want = _product_tree(req["base"][0], 5, 3, 30, 1.0, norm)
    assert _tree_paths(t) == [p for p, _ in want]
    np.testing.assert_allclose(t.scores[1:], [s for _, s in want], atol=1e-12)


def test_zero_gru_gives_depth_constant_correction():
    spec, w, req = _small_case(31, V=7, D=4, M=5, k=3, N=30, biases=False, root_std=0.0)
    w = dict(w, w_ih=np.zeros_like(w["w_ih"]), w_hh=np.zeros_like(w["w_hh"]))
    head = _head_from(spec, w)
    hid = req["hidden"][0].astype(np.float64)
    t = ref.build_tree(head, req["base"][0], hid, req["root"][0], 5, 3, 30, 1.0)
    # S stays 0, so dL_d = W2^T SiLU(W1^T [H_d; 0]) for every node of depth d
    w1, w2 = w["w1"].astype(np.float64), w["w2"].astype(np.float64)
    dl = []
    for d in range(4):
        u = np.r_[hid[d], np.zeros(spec.ds)] @ w1
        full = w2.T @ (u / (1 + np.exp(-u)))
        row = req["base"][0][d].astype(np.float64)
        ids = sorted(range(7), key=lambda v: (-row[v], v))[:5]
        dl.append(full[ids])
    want = _product_tree(req["base"][0], 5, 3, 30, 1.0, "topm", dl=dl)
    assert _tree_paths(t) == [p for p, _ in want]


def test_k1_is_the_greedy_chain():
    spec, w, req = _small_case(32, V=9, D=5, M=6, k=1, N=50)
    head = _head_from(spec, w)
    hid = req["hidden"][0].astype(np.float64)
    t = ref.build_tree(head, req["base"][0], hid, req["root"][0], 6, 1, 50, 1.0)
    # the Domino chain: update S from the drafted token, take the best corrected logit
    s, chain = req["root"][0].astype(np.float64), []
    for d in range(5):
        row = req["base"][0][d].astype(np.float64)
        ids = sorted(range(9), key=lambda v: (-row[v], v))[:6]
        z = row[ids] + ref.correction(head, hid[d], s, np.array(ids))
        tok = ids[min(range(6), key=lambda m: (-z[m], ids[m]))]
        chain.append(tok)
        s = ref.gru_step(head, s, head.emb(tok))
    assert t.n_nodes == 5                      # min(N, D): the heap runs dry
    assert t.tokens[1:] == chain
    assert t.parents[1:] == list(range(5))


def test_n1_is_the_depth1_argmax():
    spec, w, req = _small_case(33, V=9, D=3, M=9, k=9, N=1)
    head = _head_from(spec, w)
    hid = req["hidden"][0].astype(np.float64)
    t = ref.build_tree(head, req["base"][0], hid, req["root"][0], 9, 9, 1, 1.0)
    row = req["base"][0][0].astype(np.float64)
    z = row + ref.correction(head, hid[0], req["root"][0], np.arange(9))
    assert t.n_nodes == 1 and t.tokens[1] == int(np.argmax(z))


def test_vocab_permutation_relabels_tokens():
    spec, w, req = _small_case(34, V=8, D=4, M=5, k=3, N=25)
    head = _head_from(spec, w)
    hid = req["hidden"][0].astype(np.float64)
    t = ref.build_tree(head, req["base"][0], hid, req["root"][0], 5, 3, 25, 1.0)
    pi = np.random.default_rng(7).permutation(8)       # token v -> pi[v]
    inv = np.argsort(pi)
    w2 = dict(w, emb=w["emb"][inv], w2=w["w2"][:, inv])
    base2 = req["base"][0][:, inv]
    t2 = ref.build_tree(_head_from(spec, w2), base2, hid, req["root"][0], 5, 3, 25, 1.0)
    assert t2.tokens[1:] == [int(pi[v]) for v in t.tokens[1:]]
    assert t2.parents == t.parents
    np.testing.assert_allclose(t2.scores, t.scores, atol=1e-12)


@pytest.mark.parametrize("norm", ["topm", "fullv"])
def test_per_depth_logit_shift_is_invisible(norm):
    spec, w, req = _small_case(35, V=8, D=4, M=5, k=3, N=25, norm=norm)
    head = _head_from(spec, w)
    hid = req["hidden"][0].astype(np.float64)
    t = ref.build_tree(head, req["base"][0], hid, req["root"][0], 5, 3, 25, 1.0, norm)
    shifted = req["base"][0] + np.array([[3.0], [-2.0], [0.5], [7.0]], np.float32)
    t2 = ref.build_tree(head, shifted, hid, req["root"][0], 5, 3, 25, 1.0, norm)
    assert t2.tokens == t.tokens and t2.parents == t.parents
    np.testing.assert_allclose(t2.scores, t.scores, atol=1e-6)


def test_m_equals_v_makes_norms_agree_with_full_softmax():
    spec, w, req = _small_case(36, V=7, D=3, M=7, k=7, N=30)
    head = _head_from(spec, w)
    hid = req["hidden"][0].astype(np.float64)
    ta = ref.build_tree(head, req["base"][0], hid, req["root"][0], 7, 7, 30, 0.5, "topm")
    tb = ref.build_tree(head, req["base"][0], hid, req["root"][0], 7, 7, 30, 0.5, "fullv")
    assert ta.tokens == tb.tokens and ta.parents == tb.parents
    np.testing.assert_allclose(ta.scores, tb.scores, atol=1e-13)
    # node 1: full-vocabulary log-softmax of (base + dL)/T at depth 1
    row = req["base"][0][0].astype(np.float64)
    z = (row + ref.correction(head, hid[0], req["root"][0], np.arange(7))) / 0.5
    lp = torch.log_softmax(torch.from_numpy(z), 0).numpy()
    assert abs(ta.scores[1] - lp[ta.tokens[1]]) < 1e-13


def test_temperature_leaves_child_sets_unchanged():
    spec, w, req = _small_case(37, V=9, D=3, M=6, k=3, N=20)
    head = _head_from(spec, w)
    hid = req["hidden"][0].astype(np.float64)
    dep = ref.candidates(req["base"][0][0], 6, 1.0)
    dep2 = ref.candidates(req["base"][0][0], 6, 0.5)
    assert dep.cand.tolist() == dep2.cand.tolist()
    s = np.random.default_rng(8).standard_normal(spec.ds)
    a = ref.expand_scores(head, dep, hid[0], s, 3, 1.0, "topm")
    b = ref.expand_scores(head, dep2, hid[0], s, 3, 0.5, "topm")
    assert a.children == b.children


def test_neg_inf_logits_are_never_children_and_heap_runs_dry():
    spec, w, req = _small_case(38, V=6, D=3, M=4, k=4, N=50)
    base = req["base"][0].copy()
    base[:, [0, 2, 3, 5]] = -np.inf               # two finite tokens per depth
    head = _head_from(spec, w)
    t = ref.build_tree(head, base, req["hidden"][0].astype(np.float64), req["root"][0],
                       4, 4, 50, 1.0)
    assert set(t.tokens[1:]) <= {1, 4}
    assert t.n_nodes == 2 + 4 + 8                 # every finite path, then empty
    assert all(np.isfinite(t.scores))


def test_forced_ties_lowest_token_and_parent_first():
    # equal base logits and duplicate W2 columns: equal corrected logits
    spec, w, req = _small_case(39, V=4, D=2, M=4, k=2, N=6, biases=False, root_std=0.0)
    w = dict(w, w2=np.repeat(w["w2"][:, :1], 4, axis=1))
    base = np.zeros((2, 4), np.float32)
    head = _head_from(spec, w)
    t = ref.build_tree(head, base, req["hidden"][0].astype(np.float64), req["root"][0],
                       4, 2, 6, 1.0)
    assert t.tokens[1:3] == [0, 1] and t.depths[1:3] == [1, 1]
    # depth-2 children of both depth-1 nodes tie per token: parent order decides
    # (the two parents have different GRU states, so only equal scores tie)
    tail = list(zip(t.tokens[3:], t.parents[3:]))
    assert [tk for tk, _ in tail] == sorted(tk for tk, _ in tail) or len(set(t.scores[3:])) > 1


def test_m1_chain_orders_by_depth():
    spec, w, req = _small_case(40, V=5, D=4, M=1, k=1, N=10)
    head = _head_from(spec, w)
    t = ref.build_tree(head, req["base"][0], req["hidden"][0].astype(np.float64),
                       req["root"][0], 1, 1, 10, 1.0)
    assert t.scores == [0.0] * 5               # log-softmax over one candidate
    assert t.depths == [0, 1, 2, 3, 4] and t.parents == [-1, 0, 1, 2, 3]


def test_lm_head_matches_torch_and_chunks():
    rng = np.random.default_rng(9)
    H = synth.bf16_bits(rng.standard_normal((5, 16)).astype(np.float32))
    W = synth.bf16_bits(rng.standard_normal((16, 37)).astype(np.float32))
    got = ref.lm_head_logits(H, W, True, chunk=8)
    want = (torch.from_numpy(synth.bits_to_f32(H)).double()
            @ torch.from_numpy(synth.bits_to_f32(W)).double()).float().numpy()
    np.testing.assert_array_equal(got, want)


def test_certificate_accepts_oracle_and_rejects_tampering():
    spec, w, req = _small_case(41, V=8, D=4, M=5, k=3, N=25)
    head = _head_from(spec, w)
    hid = req["hidden"][0].astype(np.float64)
    t = ref.build_tree(head, req["base"][0], hid, req["root"][0], 5, 3, 25, 1.0)
    other = dict(tokens=np.array(t.tokens), parents=np.array(t.parents),
                 depths=np.array(t.depths), scores=np.array(t.scores, np.float32),
                 n_nodes=t.n_nodes)
    rep = certify.compare(t, head, hid, req["root"][0], other, 3, 1.0, "topm", 25, 1e-4)
    assert rep.exact and rep.ok and rep.max_dscore < 1e-6
    bad = {k: (v.copy() if hasattr(v, "copy") else v) for k, v in other.items()}
    bad["scores"][7] += 0.01
    assert certify.compare(t, head, hid, req["root"][0], bad, 3, 1.0, "topm", 25,
                           1e-4).failures
    short = dict(other, n_nodes=20)
    rep = certify.compare(t, head, hid, req["root"][0], short, 3, 1.0, "topm", 25, 1e-4)
    assert not rep.ok


def test_generator_is_deterministic_and_shaped():
    spec, w, req = synth.workload("tiny")
    assert req["base"].shape == (1, 7, 1024) and w["w1"].shape == (192, 32)
    synth.weights.cache_clear()
    synth.requests.cache_clear()
    _, w2, req2 = synth.workload("tiny")
    np.testing.assert_array_equal(w["w_ih"], w2["w_ih"])
    np.testing.assert_array_equal(req["base"], req2["base"])
    # boosted tokens: 1-3 per depth stand out by about +4
    assert np.all(req["base"].max(-1) > 3.0)
