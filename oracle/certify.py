"""Tree comparison and tolerance certificate (test infrastructure).

Only tests/, smoke() and bench.py's CPU-baseline leg use this module.

The pages call DominoTree's builder lossless up to floating-point
tie-breaking ("Riassunto Tecnico: DominoTree", Risultati Sperimentali) and
bit-identical to its Python reference (Componenti Core 3).  This module turns
that into a check of another builder's tree (the GPU library) against the
oracle's tree for the same request.

`compare` reports:
  * exact      -- tokens and parents equal node for node, in pop order, and
                  the same node count;
  * max_dscore -- max |score difference| over the nodes before the first
                  difference;
  * near_tie   -- the decision that produced the first difference, when the
                  oracle had a competitor within `tol` there ("pop" or
                  "topk", see `_tie_at`), else "";
  * topm_swaps -- depths where the other builder's candidate set differs from
                  the oracle's at a top-M boundary within `tol_logit` (only
                  for logits computed by an LM head on both sides; the tree is
                  then compared with the oracle's tree on the other's sets);
  * census     -- how many of the oracle's own decisions had a runner-up
                  within the tolerance (pops and top-k boundaries within
                  `tol`; with computed logits also top-M boundaries within
                  `tol_logit`).  With none, nothing excuses a difference and
                  the tree must be exact (`must_be_exact`);
  * failures   -- certificate clauses the other tree breaks, each tagged
                  with its clause name in brackets, re-evaluated with the
                  oracle's arithmetic along the other tree's own paths:
      [root]     node 0 is the root record (token -1, parent -1, depth 0,
                 score 0);
      [count]    0 <= n_nodes <= N;
      [order]    every parent precedes its child;
      [depth]    depth = parent's depth + 1, at most D;
      [dup]      no two nodes share (parent, token);
      [expand]   every parent is expandable (the root, or depth < D and
                 index < N);
      [score]    each node's score equals its path score within tol;
      [mono]     scores do not rise in pop order (by more than tol);
      [cand]     each token is a candidate of its depth;
      [topk]     each token is within tol of its parent's top-k boundary;
      [budget]   when n_nodes < N (the frontier ran dry), every expanded
                 node has all its children (its finite top-k) in the tree;
      [frontier] no left-out child that leads its parent's first candidate
                 after the top-k by at least tol beats the tree's worst node
                 by more than tol (the tree is a best-first prefix, up to
                 tol);
    and the comparison's own clauses:
      [dscore]   matched nodes' scores within tol of the oracle's;
      [mismatch] a first difference that no near tie at that decision
                 excuses.
A failure is a bug in one of the two implementations.
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
    census: dict = field(default_factory=dict)
    topm_swaps: int = 0           # depths compared on the other's candidate set

    @property
    def ok(self) -> bool:
        return not self.failures and (self.exact or bool(self.near_tie))

    @property
    def must_be_exact(self) -> bool:
        """No oracle decision had a runner-up within the tolerance."""
        return sum(self.census.values()) == 0


def census(otree: ref.Tree, tol: float, logits_computed: bool = False,
           tol_logit: float = 1e-4) -> dict:
    """Counts of the oracle's decisions whose runner-up was within tolerance.

    pop:  pops whose next heap entry was within `tol` of the popped score;
    topk: expanded nodes whose k-th and (k+1)-th corrected logits were within
          `tol` (z units, the log-prob gap at the boundary);
    topm: depths whose M-th and (M+1)-th base logits were within `tol_logit`,
          counted only when the logits were computed (an LM head): given
          logits are selected by pure comparisons on identical inputs.
    """
    n = otree.n_nodes
    out = {"pop": sum(1 for m in otree.pop_margin[:n] if m < tol),
           "topk": sum(1 for m in otree.topk_margin.values() if m < tol)}
    if logits_computed:
        out["topm"] = sum(1 for d in otree.depths_info if d.margin < tol_logit)
    return out


def evaluate(head, deps, hidden, root, tokens, parents, n: int, k: int, T: float,
             norm: str, N: int):
    """Oracle arithmetic along the given tree's own paths.

    The tree's structure must already be valid (parents precede children).
    Returns per-node path scores, the expansion of every node the builder
    expands (the root, and nodes with depth < D and index < N) and per-node
    depths.  A node whose parent has no expansion, or whose token is not a
    candidate, scores nan or -inf and is not expanded.
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
            if ex is None:      # parent not expandable: the certificate reports it
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


def _structure(tokens, parents, depths, scores, n: int, D: int, N: int) -> list:
    """Clauses root, count, order, depth, dup, expand (no arithmetic)."""
    fails = []
    if int(tokens[0]) != -1 or int(parents[0]) != -1 or int(depths[0]) != 0 \
            or float(scores[0]) != 0.0:
        fails.append("[root] node 0 is not the root record")
    if not 0 <= n <= N:
        fails.append(f"[count] n_nodes {n} outside 0..{N}")
        return fails
    seen = set()
    for i in range(1, n + 1):
        p = int(parents[i])
        if not 0 <= p < i:
            fails.append(f"[order] node {i}: parent {p} does not precede it")
            return fails
        if int(depths[i]) != int(depths[p]) + 1 or int(depths[i]) > D:
            fails.append(f"[depth] node {i}: depth {depths[i]} vs parent depth {depths[p]}")
        if (p, int(tokens[i])) in seen:
            fails.append(f"[dup] node {i}: duplicate child token {tokens[i]} of {p}")
        seen.add((p, int(tokens[i])))
        if p > 0 and (int(depths[p]) >= D or p >= N):
            fails.append(f"[expand] node {i}: parent {p} is not expandable")
    return fails


def _arithmetic(deps, tokens, parents, depths, scores, n: int, k: int, N: int, tol: float,
                sc: dict, exps: dict) -> list:
    """Clauses score, mono, cand, topk, budget, frontier on a valid structure."""
    fails = []
    for i in range(1, n + 1):
        if not abs(float(scores[i]) - sc[i]) <= tol:
            fails.append(f"[score] node {i}: score {float(scores[i])!r} vs path score {sc[i]!r}")
        if i > 1 and float(scores[i]) > float(scores[i - 1]) + tol:
            fails.append(f"[mono] node {i}: score rises in pop order")
        p = int(parents[i])
        ex = exps[p]
        dep = deps[int(depths[i]) - 1]
        hit = np.nonzero(dep.cand == int(tokens[i]))[0]
        if hit.size == 0:
            fails.append(f"[cand] node {i}: token {tokens[i]} not a candidate of depth {depths[i]}")
            continue
        order = ref.rank_desc(ex.z, dep.cand)
        kth = ex.z[order[min(k, len(order)) - 1]]
        if not ex.z[hit[0]] >= kth - tol:
            fails.append(f"[topk] node {i}: token outside its parent's top-{k} by more than tol")
    # children of expanded nodes that are not in the tree.  A builder that
    # met a top-k boundary within tol may have pushed another candidate in
    # place of one of the oracle's children, so only a child that leads the
    # first candidate after the top-k by at least tol is required.
    in_tree = {(int(parents[i]), int(tokens[i])) for i in range(1, n + 1)}
    kids_in = {}
    for i in range(1, n + 1):
        kids_in[int(parents[i])] = kids_in.get(int(parents[i]), 0) + 1
    worst = min((float(scores[i]) for i in range(1, n + 1)), default=math.inf)
    best_out = ref.NEG_INF
    for p, ex in exps.items():
        if p > n:
            continue
        dep = deps[int(depths[p])]
        order = ref.rank_desc(ex.z, dep.cand)
        next_z = ex.z[order[k]] if len(order) > k else ref.NEG_INF
        for m in ex.children:
            if (p, int(dep.cand[m])) not in in_tree and ex.z[m] - next_z >= tol:
                best_out = max(best_out, sc[p] + float(ex.logp[m]))
        if n < N and kids_in.get(p, 0) != len(ex.children):
            fails.append(f"[budget] n_nodes {n} < budget {N} while node {p} has "
                         f"{kids_in.get(p, 0)} of its {len(ex.children)} children")
    if n > 0 and best_out > worst + tol:
        fails.append(f"[frontier] a left-out child scores {best_out!r} > worst node {worst!r} + tol")
    return fails


def certify(head, deps, hidden, root, tokens, parents, depths, scores, n: int, k: int,
            T: float, norm: str, N: int, tol: float) -> list:
    """The certificate clauses (module doc) of one tree; returns the failures."""
    fails = _structure(tokens, parents, depths, scores, n, len(deps), N)
    if fails:
        return fails
    sc, exps, _ = evaluate(head, deps, hidden, root, tokens, parents, n, k, T, norm, N)
    return _arithmetic(deps, tokens, parents, depths, scores, n, k, N, tol, sc, exps)


def _same_set(a, b) -> bool:
    """Equal candidate sets (the order inside a set only numbers the slots)."""
    return np.array_equal(np.sort(np.asarray(a, dtype=np.int64)), np.sort(np.asarray(b, dtype=np.int64)))


def other_depths(otree: ref.Tree, base_rows, cand_other, T: float) -> list:
    """The oracle's per-depth candidate records, with the other builder's
    candidate set wherever it differs from the oracle's (a top-M boundary
    that the two sides' own logits settled differently).  Values are the
    oracle's logits at the other's ids; lse, margin as the oracle's; tail
    over the tokens outside the other's set."""
    out = []
    for d, dep in enumerate(otree.depths_info):
        ids = np.asarray(cand_other[d], dtype=np.int64)
        if _same_set(ids, dep.cand):
            out.append(dep)
            continue
        row = np.asarray(base_rows[d], dtype=np.float64)
        rest = np.ones(row.shape[0], bool)
        rest[ids] = False
        out.append(ref.Depth(cand=ids, base=row[ids].copy(), lse=dep.lse,
                             tail=ref.logsumexp(row[rest] / T), margin=dep.margin))
    return out


def compare(otree: ref.Tree, head, hidden, root, other: dict, k: int, T: float,
            norm: str, N: int, tol: float, logits_computed: bool = False,
            tol_logit: float = 1e-4, cand_other=None, base_rows=None) -> Report:
    """Compare another builder's tree with the oracle's (see module doc).

    `other` holds tokens, parents, depths, scores ([N + 1] each) and n_nodes.
    `logits_computed`: the base logits came from an LM head on both sides
    (each with its own rounding), so the top-M boundaries can tie too; then
    `cand_other` ([D, M], the other builder's candidates) and `base_rows`
    ([D, V], the oracle's logits) are checked: a depth whose candidate set
    differs from the oracle's must have had its boundary within `tol_logit`
    ([topm] otherwise).  Each set is then a valid choice, and the tree that
    follows from it is unique up to pop and top-k ties, so the oracle builds
    its tree again on the other's sets (`topm_swaps` counts such depths) and
    the comparison proceeds against that tree.
    """
    n_o = otree.n_nodes
    n_x = int(other["n_nodes"])
    tok, par, dep, scs = other["tokens"], other["parents"], other["depths"], other["scores"]
    deps = otree.depths_info
    cen = census(otree, tol, logits_computed, tol_logit)
    fails = []
    swaps = 0
    if cand_other is not None:
        for d, od in enumerate(deps):
            if not _same_set(cand_other[d], od.cand):
                swaps += 1
                if not (logits_computed and od.margin < tol_logit):
                    fails.append(f"[topm] depth {d + 1}: candidate set differs with no boundary "
                                 f"within tol_logit")
        if swaps and not fails:
            deps = other_depths(otree, base_rows, cand_other, T)
            otree = ref.build_tree(head, np.asarray(base_rows), hidden, root, len(deps[0].cand), k, N,
                                   T, norm, deps=deps)
            n_o = otree.n_nodes
    fails += _structure(tok, par, dep, scs, n_x, len(deps), N)
    L = max(0, min(n_o, n_x))
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
    if not fails:
        sc, exps, _ = evaluate(head, deps, hidden, root, tok, par, n_x, k, T, norm, N)
        fails = _arithmetic(deps, tok, par, dep, scs, n_x, k, N, tol, sc, exps)
        if not exact:
            near = _tie_at(otree, tok, par, dep, n_x, first, sc, exps, tol)
    if not exact and not near:
        fails.append(f"[mismatch] first difference at node {first} with no oracle decision "
                     f"within tol there")
    if maxd > tol:
        fails.append(f"[dscore] matched-node score difference {maxd!r} > tol")
    return Report(exact=exact, n_oracle=n_o, n_other=n_x, first_mismatch=first,
                  near_tie=near, max_dscore=maxd, failures=fails, census=cen, topm_swaps=swaps)


def _tie_at(otree: ref.Tree, tokens, parents, depths, n_x: int, first: int, sc: dict,
            exps: dict, tol: float) -> str:
    """The near tie that excuses the first difference, or "".

    Nodes 1..first-1 are the same in both trees, so both builders took the
    same pops up to there and expanded the same nodes the same way (in the
    oracle's arithmetic).  Let A be the oracle's node `first` and B the other
    tree's.  The difference is excused only when the two are competitors
    within the tolerance in the oracle's own arithmetic, |score(A) -
    score(B)| < tol (B scored along its own path), and then by the decision
    that separates them:
      * "pop"  -- B is one of the oracle's children of its parent, so both
                  were in the oracle's heap at this pop and the oracle's pop
                  margin there is below tol;
      * "topk" -- B is not one of them: B's parent (a node both trees share)
                  had a top-k boundary within tol, where the other builder
                  kept B instead.
    (A top-M boundary is settled before the tree is built: see `compare`.)
    Differing node counts (one tree a prefix of the other) are never excused:
    the count depends on no floating-point decision.
    """
    n_o = otree.n_nodes
    if first < 1 or first > n_o or first > n_x:
        return ""
    pb, tb = int(parents[first]), int(tokens[first])
    db = int(depths[first])
    dep = otree.depths_info[db - 1]
    if not np.any(dep.cand == tb) or not abs(otree.scores[first] - sc[first]) < tol:
        return ""
    ex = exps.get(pb)
    if ex is None:
        return ""
    kids = {int(dep.cand[m]) for m in ex.children}
    if tb in kids:
        return "pop" if otree.pop_margin[first - 1] < tol else ""
    return "topk" if otree.topk_margin.get(pb, math.inf) < tol else ""
