"""Pins of the comparison layer (oracle/certify.py).

Each certificate clause is shown to fire on a tree tampered in the one way it
guards against, and the near-tie excuse is shown to accept only a difference
at a decision the oracle itself took within the tolerance: a genuine pop or
top-k near tie is excused, the same difference behind a larger margin fails.
The tampered trees are built from the oracle's own tree and its frontier, so
every other clause stays satisfied where the test says so.
"""
import re

import numpy as np
import pytest

from oracle import certify, ref
from workloads import synth

K, M, N, T = 3, 5, 25, 1.0


def _case(seed):
    spec = synth.small(f"s{seed}", V=8, D=4, M=M, k=K, N=N, T=T, group=1000 + seed,
                       norm="topm", wdtype="f32", biases=True, root_std=0.5)
    spec, w, req = synth.workload(spec)
    head = ref.make_head(w, False, False)
    hid = req["hidden"][0].astype(np.float64)
    root = req["root"][0]
    t = ref.build_tree(head, req["base"][0], hid, root, M, K, N, T)
    return head, hid, root, t


def _other(t):
    return dict(tokens=np.array(t.tokens), parents=np.array(t.parents),
                depths=np.array(t.depths), scores=np.array(t.scores, np.float32),
                n_nodes=t.n_nodes)


def _cmp(case, other, tol=1e-4):
    head, hid, root, t = case
    return certify.compare(t, head, hid, root, other, K, T, "topm", N, tol)


def _codes(rep):
    return {m for f in rep.failures for m in re.findall(r"^\[(\w+)\]", f)}


def _frontier(case):
    """Left-out children of the oracle tree's expanded nodes, best first by
    the heap's total order: (score, depth, token, parent, slot, z gap to the
    next child)."""
    head, hid, root, t = case
    sc, exps, _ = certify.evaluate(head, t.depths_info, hid, root, t.tokens, t.parents,
                                   t.n_nodes, K, T, "topm", N)
    in_tree = set(zip(t.parents[1:], t.tokens[1:]))
    out = []
    for p, ex in exps.items():
        dep = t.depths_info[t.depths[p]]
        for m in range(M):
            tok = int(dep.cand[m])
            if (p, tok) not in in_tree:
                out.append((sc[p] + float(ex.logp[m]), t.depths[p] + 1, tok, p, m,
                            m in ex.children))
    out.sort(key=lambda e: (-e[0], e[1], e[2], e[3]))
    return out


def _replace(other, i, tok, par, dep, score):
    o = {k: (v.copy() if hasattr(v, "copy") else v) for k, v in other.items()}
    o["tokens"][i], o["parents"][i], o["depths"][i], o["scores"][i] = tok, par, dep, score
    return o


@pytest.fixture(scope="module")
def case77():
    return _case(77)


def test_oracle_tree_is_exact_and_certified(case77):
    rep = _cmp(case77, _other(case77[3]))
    assert rep.exact and rep.ok and not rep.failures and rep.max_dscore < 1e-6
    # census at a tiny tolerance: no decision of this tree is that close
    assert rep.must_be_exact and rep.census == {"pop": 0, "topk": 0}


def test_root_clause(case77):
    o = _other(case77[3])
    o["scores"][0] = 0.5
    assert "root" in _codes(_cmp(case77, o))


def test_count_clause_and_no_tree(case77):
    o = dict(_other(case77[3]), n_nodes=N + 1)
    assert "count" in _codes(_cmp(case77, o))
    rep = _cmp(case77, dict(_other(case77[3]), n_nodes=-1))      # a failed build
    assert "count" in _codes(rep) and rep.near_tie == "" and not rep.ok


def test_order_clause(case77):
    o = _other(case77[3])
    o["parents"][5] = 7
    assert "order" in _codes(_cmp(case77, o))


def test_depth_clause(case77):
    o = _other(case77[3])
    o["depths"][4] += 1
    assert "depth" in _codes(_cmp(case77, o))


def test_dup_clause(case77):
    t = case77[3]
    o = _replace(_other(t), t.n_nodes, t.tokens[1], t.parents[1], t.depths[1],
                 t.scores[t.n_nodes])
    assert "dup" in _codes(_cmp(case77, o))


def test_expand_clause(case77):
    # a node hung below a depth-D node
    t = case77[3]
    leaf = next(i for i in range(1, t.n_nodes) if t.depths[i] == 4)
    o = _replace(_other(t), t.n_nodes, 0, leaf, 5, t.scores[t.n_nodes])
    assert "expand" in _codes(_cmp(case77, o))


def test_score_and_dscore_clauses(case77):
    o = _other(case77[3])
    o["scores"][7] += 0.01
    assert {"score", "dscore"} <= _codes(_cmp(case77, o))


def test_mono_clause_and_mismatch_behind_a_large_margin(case77):
    # two leaves swapped in pop order where the oracle's pop margin is large
    t = case77[3]
    used = set(t.parents)
    j = max((i for i in range(1, t.n_nodes) if i not in used and i + 1 not in used),
            key=lambda i: t.pop_margin[i - 1])
    assert t.pop_margin[j - 1] > 1.0
    o = _other(t)
    for key in ("tokens", "parents", "depths", "scores"):
        o[key][[j, j + 1]] = o[key][[j + 1, j]]
    rep = _cmp(case77, o, tol=0.5)
    assert {"mono", "mismatch"} <= _codes(rep) and rep.near_tie == ""


def test_cand_clause(case77):
    t = case77[3]
    n = t.n_nodes
    dep = t.depths_info[t.depths[n] - 1]
    outsider = next(v for v in range(8) if v not in dep.cand)
    o = _replace(_other(t), n, outsider, t.parents[n], t.depths[n], t.scores[n])
    assert "cand" in _codes(_cmp(case77, o))


def test_topk_clause(case77):
    # the last node replaced by a candidate of its parent far outside the
    # parent's top-k, carrying its true path score
    t = case77[3]
    n = t.n_nodes
    far = [e for e in _frontier(case77) if e[3] == t.parents[n] and not e[5]]
    s, d, tok, p, m, _ = far[-1]
    o = _replace(_other(t), n, tok, p, d, s)
    rep = _cmp(case77, o, tol=1e-3)
    assert "topk" in _codes(rep) and "score" not in _codes(rep)


def test_budget_clause(case77):
    # the build stopping one node early although the frontier is not empty
    o = dict(_other(case77[3]), n_nodes=N - 1)
    rep = _cmp(case77, o)
    assert "budget" in _codes(rep) and "mismatch" in _codes(rep)


def test_frontier_clause(case77):
    # the last node replaced by the worst legal child, with its true score:
    # the oracle's last node, now left out, beats it by far
    t = case77[3]
    worst = [e for e in _frontier(case77) if e[5]][-1]
    s, d, tok, p, m, _ = worst
    o = _replace(_other(t), t.n_nodes, tok, p, d, s)
    rep = _cmp(case77, o, tol=1e-3)
    assert "frontier" in _codes(rep) and "score" not in _codes(rep) \
        and "topk" not in _codes(rep)


def test_pop_near_tie_excused_only_within_tol(case77):
    # the last pop: the oracle took node N over the best left-out child C by
    # its pop margin; a builder that took C instead differs by a pop tie
    t = case77[3]
    s, d, tok, p, m, _ = [e for e in _frontier(case77) if e[5]][0]   # the heap's top
    gap = t.pop_margin[N - 1]
    assert abs((t.scores[N] - s) - gap) < 1e-12 and 0.1 < gap < 0.2
    o = _replace(_other(t), N, tok, p, d, s)
    rep = _cmp(case77, o, tol=0.2)
    assert rep.ok and not rep.exact and rep.near_tie == "pop" and rep.first_mismatch == N
    assert not rep.must_be_exact and rep.census["pop"] >= 1
    rep = _cmp(case77, o, tol=0.1)
    assert not rep.ok and rep.near_tie == "" and "mismatch" in _codes(rep)


def test_topk_near_tie_excused_only_within_tol():
    # seed 78: the oracle's last node is the k-th child of its parent, whose
    # top-k boundary margin (0.253) is below its last pop margin (0.281).  A
    # builder that kept the (k+1)-th candidate instead differs by a top-k tie
    case = _case(78)
    t = case[3]
    n = t.n_nodes
    p = t.parents[n]
    gap = t.topk_margin[p]
    assert 0.25 < gap < t.pop_margin[n - 1] < 0.29
    nxt = [e for e in _frontier(case) if e[3] == p and not e[5]][0]
    s, d, tok, _, m, _ = nxt
    assert abs((t.scores[n] - s) - gap) < 1e-12
    o = _replace(_other(t), n, tok, p, d, s)
    rep = _cmp(case, o, tol=0.27)
    assert rep.ok and rep.near_tie == "topk", rep
    rep = _cmp(case, o, tol=0.2)
    assert not rep.ok and rep.near_tie == "" and {"mismatch", "topk"} <= _codes(rep)


def test_census_counts_exact_ties():
    # the hand-worked tie fixture: equal scores everywhere
    import json
    import os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_tree_ties.json")))
    V, D, ds = fx["V"], fx["D"], 2
    base = np.array(fx["logits"], np.float64)
    w = {"emb": np.zeros((V, 2), np.float32), "w_ih": np.zeros((3 * ds, 2), np.float32),
         "w_hh": np.zeros((3 * ds, ds), np.float32), "w1": np.zeros((2 + ds, 2), np.float32),
         "w2": np.zeros((2, V), np.float32), "b_ih": None, "b_hh": None}
    head = ref.make_head(w, False, False)
    t = ref.build_tree(head, base, np.zeros((D, 2)), np.zeros(ds), fx["M"], fx["k"], fx["N"],
                       fx["T"])
    assert t.tokens == fx["expected"]["tokens"]
    c = certify.census(t, 1e-9)
    assert c["pop"] > 0
    assert "topm" not in c and "topm" in certify.census(t, 1e-9, logits_computed=True)


def test_length_difference_is_never_excused(case77):
    t = case77[3]
    o = dict(_other(t), n_nodes=N - 1)
    rep = _cmp(case77, o, tol=10.0)
    assert rep.near_tie == "" and not rep.ok


def test_topm_near_tie_with_computed_logits():
    # two builders whose own logits settle a depth-1 top-M boundary (within
    # 1e-5 in the oracle's logits) differently: the other tree holds the
    # (M+1)-th token where the oracle holds the M-th, and everything that
    # follows from its own correction.  Accepted only for computed logits and
    # a boundary within tol_logit, by comparison with the oracle's tree on the
    # other's candidate sets.
    spec = synth.small("s_topm", V=8, D=3, M=3, k=3, N=10, T=1.0, group=1990, norm="topm", wdtype="f32",
                       biases=True, root_std=0.5)
    spec, w, req = synth.workload(spec)
    head = ref.make_head(w, False, False)
    hid = req["hidden"][0].astype(np.float64)
    root = req["root"][0]
    base = req["base"][0].copy()
    order = ref.rank_desc(base[0], np.arange(8))
    a, b = int(order[2]), int(order[3])               # the M-th and (M+1)-th of depth 1
    base[0, b] = base[0, a] - np.float32(1e-5)
    other_base = base.copy()
    other_base[0, b] = base[0, a] + np.float32(1e-5)  # the other side's logits swap them
    t = ref.build_tree(head, base, hid, root, 3, 3, 10, 1.0)
    x = ref.build_tree(head, other_base, hid, root, 3, 3, 10, 1.0)
    assert t.tokens != x.tokens
    other = _other(x)
    cand_x = np.array([d.cand for d in x.depths_info])

    def cmp(**kw):
        return certify.compare(t, head, hid, root, other, 3, 1.0, "topm", 10, 1e-3, **kw)

    rep = cmp(logits_computed=True, tol_logit=1e-4, cand_other=cand_x, base_rows=base)
    assert rep.ok and rep.exact and rep.topm_swaps == 1 and rep.max_dscore < 1e-3, rep
    assert rep.census.get("topm") == 1
    # a boundary farther than tol_logit does not excuse it
    rep = cmp(logits_computed=True, tol_logit=1e-6, cand_other=cand_x, base_rows=base)
    assert not rep.ok and "topm" in _codes(rep)
    # nor do given logits, where the sets must be equal
    rep = cmp(logits_computed=False, cand_other=cand_x, base_rows=base)
    assert not rep.ok and "topm" in _codes(rep)
    # and without the other's candidate sets the trees simply differ
    rep = cmp(logits_computed=True, tol_logit=1e-4)
    assert not rep.ok


def test_candidate_order_inside_a_set_is_not_a_swap():
    # the same candidate set listed in another order (two values inside the
    # set within the other side's rounding) is no top-M difference at all
    head, hid, root, t = _case(77)
    cand_x = np.array([d.cand for d in t.depths_info])
    cand_x[0, [0, 1]] = cand_x[0, [1, 0]]
    rep = certify.compare(t, head, hid, root, _other(t), K, T, "topm", N, 1e-4, logits_computed=False,
                          cand_other=cand_x, base_rows=np.zeros((4, 8)))
    assert rep.ok and rep.exact and rep.topm_swaps == 0
