"""Tree comparison and tolerance certificate (test infrastructure).

Only tests/, smoke() and bench.py's CPU-baseline leg use this module.

Given a tree produced elsewhere (the GPU library) and the oracle's tree for
the same request, `compare` reports:
  * exact   -- tokens and parents equal node for node, in pop order;
  * scores  -- max |score difference| over the nodes that match;
  * near_tie -- at the first mismatch, the oracle had a competitor within
               `tol` (a pop, a top-k boundary or a top-M boundary);
  * certificate failures on the other tree, re-evaluated with the oracle's
    arithmetic along its own paths:
      - node 0 is the root; parents precede children; depth = parent + 1;
        no duplicate (parent, token) pairs; n_nodes == N unless the frontier
        is empty;
      - each node's score equals its path score within tol;
      - each node's token is within tol of its parent's top-k boundary;
      - scores are non-increasing in pop order (within tol);
      - no child left out of the tree beats the tree's worst node by more
        than tol (the tree is a best-first prefix, up to tol).
A certificate failure is a bug in one of the two implementations.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import ref


@dataclass
class Report:
    exact: bool
    n_oracle: int
    n_other: int
    first_mismatch: int           # -1 if exact
    near_tie: str                 # "" or the decision type that tied
    max_dscore: float             # over nodes matching the oracle's
    failures: list = field(default_factory=list)

    @property
    def ok(self) -> bool:
        return not self.failures and (self.exact or bool(self.near_tie))


def evaluate(head, deps, hidden, root, tokens, parents, n: int, k: int, T: float,
             norm: str, N: int):
    """Oracle arithmetic along the given tree's own paths.

    Returns per-node path scores, per-node expansions (for nodes the builder
    expands: depth < D and index < N) and per-node states.
    """
    D = len(deps)
    states = {0: np.asarray(root, dtype=np.float64)}
    score = {0: 0.0}
    exps = {}
    depth = {0: 0}
    for i in range(0, n + 1):
        if i > 0:
            p = int(parents[i])
            tok = int(tokens[i])
            depth[i] = depth[p] + 1
            ex = exps.get(p)
            if ex is None:      # parent not expandable: certificate reports it
                score[i] = math.nan
                continue
            hit = np.nonzero(deps[depth[i] - 1].cand == tok)[0]
            score[i] = score[p] + float(ex.logp[hit[0]]) if hit.size else ref.NEG_INF
            if depth[i] < D and i < N and hit.size:
                states[i] = ref.gru_step(head, states[p], head.emb(tok))
        if depth[i] < D and (i < N or i == 0) and i in states:
            d = depth[i] + 1
            exps[i] = ref.expand_scores(head, deps[d - 1], hidden[d - 1], states[i], k, T,
                                        norm)
    return score, exps, depth


def certify(head, deps, hidden, root, tokens, parents, depths, scores, n: int, k: int,
            T: float, norm: str, N: int, tol: float) -> list:
    fails = []
    D = len(deps)
    if int(tokens[0]) != -1 or int(parents[0]) != -1 or int(depths[0]) != 0 \
            or float(scores[0]) != 0.0:
        fails.append("root record")
    seen = set()
    for i in range(1, n + 1):
        p = int(parents[i])
        if not (0 <= p < i):
            fails.append(f"node {i}: parent {p} does not precede it")
            return fails
        if int(depths[i]) != int(depths[p]) + 1 or int(depths[i]) > D:
            fails.append(f"node {i}: depth {depths[i]} vs parent depth {depths[p]}")
        if (p, int(tokens[i])) in seen:
            fails.append(f"node {i}: duplicate child token {tokens[i]} of {p}")
        seen.add((p, int(tokens[i])))
        if p > 0 and (int(depths[p]) >= D or p >= N):
            fails.append(f"node {i}: parent {p} is not expandable")
    if fails:
        return fails
    sc, exps, _ = evaluate(head, deps, hidden, root, tokens, parents, n, k, T, norm, N)
    for i in range(1, n + 1):
        if not abs(float(scores[i]) - sc[i]) <= tol:
            fails.append(f"node {i}: score {float(scores[i])!r} vs path score {sc[i]!r}")
        if i > 1 and float(scores[i]) > float(scores[i - 1]) + tol:
            fails.append(f"node {i}: score rises in pop order")
        p = int(parents[i])
        ex = exps.get(p)
        if ex is None:
            fails.append(f"node {i}: parent {p} has no valid path")
            continue
        dep = deps[int(depths[i]) - 1]
        m = int(np.nonzero(dep.cand == int(tokens[i]))[0][0]) \
            if np.any(dep.cand == int(tokens[i])) else -1
        if m < 0:
            fails.append(f"node {i}: token {tokens[i]} not a candidate of depth {depths[i]}")
            continue
        order = ref.rank_desc(ex.z, dep.cand)
        kth = ex.z[order[min(k, len(order)) - 1]]
        if not ex.z[m] >= kth - tol:
            fails.append(f"node {i}: token outside its parent's top-{k} by more than tol")
    # frontier: legal children of expanded nodes that are not in the tree
    in_tree = {(int(parents[i]), int(tokens[i])) for i in range(1, n + 1)}
    worst = min((float(scores[i]) for i in range(1, n + 1)), default=math.inf)
    best_out = ref.NEG_INF
    for p, ex in exps.items():
        if p > n:
            continue
        dep = deps[int(depths[p])]
        for m in ex.children:
            if (p, int(dep.cand[m])) not in in_tree:
                best_out = max(best_out, sc[p] + float(ex.logp[m]))
    if n < N and best_out != ref.NEG_INF:
        fails.append(f"n_nodes {n} < budget {N} while the frontier is not empty")
    if n > 0 and best_out > worst + tol:
        fails.append(f"a left-out child scores {best_out!r} > worst node {worst!r} + tol")
    return fails


def compare(otree: ref.Tree, head, hidden, root, other: dict, k: int, T: float,
            norm: str, N: int, tol: float) -> Report:
    """Compare another builder's tree with the oracle's (see module doc)."""
    n_o = otree.n_nodes
    n_x = int(other["n_nodes"])
    tok, par, dep, scs = other["tokens"], other["parents"], other["depths"], other["scores"]
    L = min(n_o, n_x)
    first = -1
    maxd = 0.0
    for i in range(1, L + 1):
        if int(tok[i]) != otree.tokens[i] or int(par[i]) != otree.parents[i]:
            first = i
            break
        maxd = max(maxd, abs(float(scs[i]) - otree.scores[i]))
    exact = first < 0 and n_o == n_x
    if first < 0 and not exact:
        first = L + 1
    near = ""
    if not exact:
        near = _tie_at(otree, first, tol)
    fails = certify(head, otree.depths_info, hidden, root, tok, par, dep, scs, n_x, k, T,
                    norm, N, tol)
    if not exact and not near:
        fails.append(f"mismatch at node {first} with no oracle decision within tol")
    if maxd > tol:
        fails.append(f"matched-node score difference {maxd!r} > tol")
    return Report(exact=exact, n_oracle=n_o, n_other=n_x, first_mismatch=first,
                  near_tie=near, max_dscore=maxd, failures=fails)


def _tie_at(otree: ref.Tree, first: int, tol: float) -> str:
    """Which oracle decision at node `first` had a competitor within tol.

    Every node before `first` matched, so the trees part at the pop that
    produced node `first`: either the oracle's heap held an entry within tol
    of the one it popped, or a node expanded earlier pushed a different child
    set (a top-k boundary within tol), or the candidate sets differ (a top-M
    boundary within tol, possible only when the base logits are computed).
    """
    if first - 1 < len(otree.pop_margin) and otree.pop_margin[first - 1] < tol:
        return "pop"
    for i, mg in otree.topk_margin.items():
        if i < first and mg < tol:
            return "topk"
    for d in otree.depths_info:
        if d.margin < tol:
            return "topm"
    return ""
