"""CPU oracle for DominoTree's conditional best-first draft-tree builder.

TEST INFRASTRUCTURE.  Only tests/, the package entry's smoke() and bench.py's
CPU-baseline leg may import or run this module.  The GPU library never does,
and this module imports nothing from it.

It is written for a reader who checks it against the pages by eye: plain
NumPy float64, one request at a time, a `heapq` best-first loop, no blocking,
fusion or reordering.  Citations name the page and its section:

  [Domino, Method]     "Domino：在投机解码中将因果建模与自回归草稿解耦",
                       section 核心方法 (the Domino head: GRU causal encoder and
                       low-rank logit-space correction, final logits = base + dL)
  [Domino, Steps]      same page, section 方法步骤详情 (base logits from the
                       frozen LM head over the draft block; inference updates the
                       causal state from the previously drafted token)
  [DominoTree, Core 1] "Riassunto Tecnico: DominoTree", Componenti Core 1
                       (best-first max-heap keyed by cumulative path log-prob;
                       children scored by re-running the GRU correction along
                       the node's own path; H_d shared by all paths)
  [DominoTree, Core 2] same page, Componenti Core 2 (correction restricted to
                       the per-depth top-M marginal candidates -- the r x M
                       slice of W2 -- before picking the top-k children)
  [DominoTree, Core 4] same page, Componenti Core 4 (fixed node budget)

Readings of points the pages leave open (each is also listed in the design
notes of the repository):
  * GRU form: the torch.nn.GRUCell convention -- gate rows (reset, update,
    new); the reset gate multiplies (W_hn h + b_hn); h' = (1-z) n + z h.
  * A child at depth d uses H_d and its parent's state; the root's children use
    the caller's root state with no GRU step at the root.
  * Normalisation "topm" (default): log-softmax over the M corrected
    candidate logits.  "fullv": the normaliser also holds the log-sum-exp of
    the uncorrected base logits of the tokens outside the top-M ("tail").
  * Temperature divides (base + dL) before the normalisation.
  * Candidates: the M largest base logits of the depth, ties to the lowest
    token id, +0 and -0 equal.  Children: the k largest corrected logits,
    ties to the lowest token id; a candidate with a -inf log-prob is never a
    child.
  * Heap order (a total order): score desc, depth asc, token asc, parent's
    node index asc.  Scores are natural-log sums of the path's log-probs.
  * Budget N counts non-root nodes; a node joins the tree when popped; the
    N-th popped node and depth-D nodes are not expanded; the build stops after
    N pops or when the heap is empty.
  * bf16 workloads: weights, embeddings and hidden states are bf16 values
    (exact here in float64); the state S is carried at full precision and
    rounded to bf16 (nearest-even, via fp32) only where it is a matrix
    operand (W_hh S and the S half of W1) when `act_bf16` is set.  The
    elementwise terms use the unrounded state.
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, field

import numpy as np

NEG_INF = float("-inf")


# ----------------------------------------------------------------------------
# elementary pieces


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """The float64 values denoted by stored bf16 bit patterns."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to fp32, then to the nearest bf16 (ties to even); return float64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    """SiLU, the correction head's activation [Domino, Method]."""
    return x * sigmoid(x)


def logsumexp(x) -> float:
    """log sum exp over a 1-D array; -inf for an empty or all -inf input."""
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return NEG_INF
    m = float(np.max(x))
    if m == NEG_INF:
        return NEG_INF
    return m + math.log(float(np.sum(np.exp(x - m))))


def rank_desc(values: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Positions of `values` sorted by (value desc, id asc); +0 == -0."""
    v = np.asarray(values, dtype=np.float64) + 0.0   # -0.0 + 0.0 == +0.0
    return np.lexsort((np.asarray(ids), -v))


# ----------------------------------------------------------------------------
# the Domino head, step by step


@dataclass
class Head:
    """Domino head weights as float64 arrays (bf16 inputs widened exactly).

    emb rows and w2 columns are widened on demand (the tables are large).
    """
    emb_store: np.ndarray      # [V, e] fp32 or bf16 bits
    w_ih: np.ndarray           # [3 ds, e]
    w_hh: np.ndarray           # [3 ds, ds]
    b_ih: np.ndarray           # [3 ds]
    b_hh: np.ndarray           # [3 ds]
    w1: np.ndarray             # [h + ds, r]
    w2_store: np.ndarray       # [r, V] fp32 or bf16 bits
    act_bf16: bool
    bf16: bool

    @property
    def ds(self):
        return self.w_hh.shape[1]

    def emb(self, v: int) -> np.ndarray:
        row = self.emb_store[v]
        return bf16_values(row) if self.bf16 else row.astype(np.float64)

    def w2_cols(self, ids) -> np.ndarray:
        cols = self.w2_store[:, np.asarray(ids)]
        return bf16_values(cols) if self.bf16 else cols.astype(np.float64)


def make_head(w: dict, bf16: bool, act_bf16: bool) -> Head:
    wide = bf16_values if bf16 else (lambda a: np.asarray(a, dtype=np.float64))
    ds3 = w["w_hh"].shape[0]
    zeros = np.zeros(ds3)
    return Head(
        emb_store=w["emb"],
        w_ih=wide(w["w_ih"]),
        w_hh=wide(w["w_hh"]),
        b_ih=zeros if w["b_ih"] is None else np.asarray(w["b_ih"], np.float64),
        b_hh=zeros if w["b_hh"] is None else np.asarray(w["b_hh"], np.float64),
        w1=wide(w["w1"]),
        w2_store=w["w2"],
        act_bf16=act_bf16,
        bf16=bf16,
    )


def operand(head: Head, s: np.ndarray) -> np.ndarray:
    """The state as a matrix operand: bf16-rounded when act_bf16 is set."""
    return round_bf16(s) if head.act_bf16 else s


def gru_step(head: Head, s: np.ndarray, x: np.ndarray) -> np.ndarray:
    """One step of the causal encoder S' = GRU(S, E[token]) [Domino, Method].

    torch.nn.GRUCell equations; the gate rows of w_ih / w_hh are (r, z, n).
    """
    ds = head.ds
    gi = head.w_ih @ x + head.b_ih
    gh = head.w_hh @ operand(head, s) + head.b_hh
    r = sigmoid(gi[:ds] + gh[:ds])
    z = sigmoid(gi[ds:2 * ds] + gh[ds:2 * ds])
    n = np.tanh(gi[2 * ds:] + r * gh[2 * ds:])
    return (1.0 - z) * n + z * s


def correction(head: Head, h_d: np.ndarray, s: np.ndarray, cand: np.ndarray) -> np.ndarray:
    """dL on the candidate columns only: W2[:, cand]^T SiLU(W1^T [H_d; S]).

    [Domino, Method] for the head; [DominoTree, Core 2] for the restriction
    to the candidate columns.
    """
    u = np.concatenate([h_d, operand(head, s)]) @ head.w1
    a = silu(u)
    return head.w2_cols(cand).T @ a


# ----------------------------------------------------------------------------
# per-depth candidates


@dataclass
class Depth:
    cand: np.ndarray      # [M] token ids, sorted by (base desc, id asc)
    base: np.ndarray      # [M] their base logits (float64 of the fp32 inputs)
    lse: float            # log-sum-exp over the whole vocabulary of base/T
    tail: float           # log-sum-exp of base/T over tokens outside cand
    margin: float         # base[M-1] - next best base logit (inf if M == V)


def candidates(row: np.ndarray, M: int, T: float) -> Depth:
    """Top-M of one depth's base logits [DominoTree, Core 2]."""
    row = np.asarray(row, dtype=np.float64)
    V = row.shape[0]
    order = rank_desc(row, np.arange(V))
    cand = order[:M]
    rest = order[M:]
    margin = math.inf
    if rest.size:
        a, b = float(row[cand[-1]]), float(row[rest[0]])
        margin = 0.0 if a == b else a - b
    return Depth(cand=cand.astype(np.int64), base=row[cand].copy(),
                 lse=logsumexp(row / T), tail=logsumexp(row[rest] / T), margin=margin)


# ----------------------------------------------------------------------------
# scoring one expansion


@dataclass
class Expansion:
    z: np.ndarray         # [M] corrected, temperature-scaled logits
    logp: np.ndarray      # [M] normalised log-probs
    children: list        # slots m of the children, best first
    margin: float         # z gap between the last child and the first non-child


def expand_scores(head: Head, dep: Depth, h_d: np.ndarray, s: np.ndarray, k: int,
                  T: float, norm: str) -> Expansion:
    """Score the M candidates of the next depth given the parent's state.

    Final logits are base + dL [Domino, Method]; divided by T, then
    log-softmaxed over the candidates (topm) or over the candidates plus the
    base tail (fullv); the k best become children [DominoTree, Core 2].
    """
    dl = correction(head, h_d, s, dep.cand)
    z = (dep.base + dl) / T
    if norm == "topm":
        lz = logsumexp(z)
    elif norm == "fullv":
        lz = logsumexp(np.append(z, dep.tail))
    else:
        raise ValueError(norm)
    logp = z - lz if lz != NEG_INF else np.full_like(z, NEG_INF)
    order = rank_desc(z, dep.cand)
    kids = [int(m) for m in order[:k] if logp[m] != NEG_INF]
    margin = math.inf
    if len(order) > k and np.isfinite(z[order[k - 1]]):
        margin = float(z[order[k - 1]] - z[order[k]])
    return Expansion(z=z, logp=logp, children=kids, margin=margin)


# ----------------------------------------------------------------------------
# the best-first builder


@dataclass
class Tree:
    tokens: list = field(default_factory=list)    # node 0 = root (-1)
    parents: list = field(default_factory=list)
    depths: list = field(default_factory=list)
    scores: list = field(default_factory=list)    # float64
    slots: list = field(default_factory=list)     # candidate slot m (-1 root)
    pop_margin: list = field(default_factory=list)   # per popped node: gap to next heap entry
    topk_margin: dict = field(default_factory=dict)  # node -> z gap at its top-k boundary
    depths_info: list = field(default_factory=list)  # per depth d=1..D: Depth

    @property
    def n_nodes(self) -> int:
        return len(self.tokens) - 1


def build_tree(head: Head, base: np.ndarray, hidden: np.ndarray, root: np.ndarray,
               M: int, k: int, N: int, T: float, norm: str = "topm", deps=None) -> Tree:
    """Best-first conditional tree for one request [DominoTree, Core 1, 2, 4].

    base   [D, V] base logits (fp32 values)
    hidden [D, h] backbone hidden states H_1..H_D (float64 values)
    root   [ds]   the root GRU state
    deps   per-depth candidate records to use instead of selecting them from
           `base` (a candidate set that another implementation's own rounding
           of computed logits settled differently at a near tie)
    """
    D = base.shape[0]
    if deps is None:
        deps = [candidates(base[d], M, T) for d in range(D)]
    t = Tree(depths_info=deps)
    t.tokens.append(-1)
    t.parents.append(-1)
    t.depths.append(0)
    t.scores.append(0.0)
    t.slots.append(-1)
    states = {0: np.asarray(root, dtype=np.float64)}
    heap: list = []

    def expand(i: int):
        d = t.depths[i] + 1                    # depth of the children (1-based)
        ex = expand_scores(head, deps[d - 1], hidden[d - 1], states[i], k, T, norm)
        t.topk_margin[i] = ex.margin
        for m in ex.children:
            tok = int(deps[d - 1].cand[m])
            heapq.heappush(heap, (-(t.scores[i] + float(ex.logp[m])), d, tok, i, m))

    expand(0)
    while t.n_nodes < N and heap:
        negs, d, tok, par, m = heapq.heappop(heap)
        t.pop_margin.append((-negs) - (-heap[0][0]) if heap else math.inf)
        i = len(t.tokens)
        t.tokens.append(tok)
        t.parents.append(par)
        t.depths.append(d)
        t.scores.append(-negs)
        t.slots.append(m)
        if d < D and i < N:
            states[i] = gru_step(head, states[par], head.emb(tok))
            expand(i)
    return t


def path_of(tree_tokens, tree_parents, i: int) -> list:
    """Tokens on the root->node path of node i (root excluded)."""
    out = []
    while i > 0:
        out.append(int(tree_tokens[i]))
        i = int(tree_parents[i])
    return out[::-1]


def score_path(head: Head, deps: list, hidden: np.ndarray, root: np.ndarray,
               path: list, T: float, norm: str) -> tuple[float, list]:
    """Re-evaluate a path's cumulative log-prob with no heap.

    Walks the path from the root, advancing the GRU state by each token and
    scoring each token against the correction of its depth.  Returns the
    cumulative score and, per depth, the expansion used (for the certificate).
    A token that is not among the depth's candidates scores -inf.
    """
    s = np.asarray(root, dtype=np.float64)
    total = 0.0
    exps = []
    for j, tok in enumerate(path):
        dep = deps[j]
        ex = expand_scores(head, dep, hidden[j], s, len(dep.cand), T, norm)
        exps.append(ex)
        hit = np.nonzero(dep.cand == tok)[0]
        if hit.size == 0:
            return NEG_INF, exps
        total += float(ex.logp[hit[0]])
        if j + 1 < len(path):
            s = gru_step(head, s, head.emb(tok))
    return total, exps


# ----------------------------------------------------------------------------
# the LM head for the pipeline that starts from hidden states


def lm_head_logits(hidden_bits_or_f32: np.ndarray, w_lm_store: np.ndarray, bf16: bool,
                   rows=None, chunk: int = 8192) -> np.ndarray:
    """Base logits L = H W_lm [Domino, Steps], float64 products rounded to fp32.

    hidden [R, h]; w_lm [h, V]; `rows` selects a subset of hidden rows.
    Computed over vocabulary chunks to bound memory.
    """
    wide = bf16_values if bf16 else (lambda a: np.asarray(a, dtype=np.float64))
    H = wide(hidden_bits_or_f32 if rows is None else hidden_bits_or_f32[rows])
    V = w_lm_store.shape[1]
    out = np.empty((H.shape[0], V), np.float32)
    for c0 in range(0, V, chunk):
        c1 = min(V, c0 + chunk)
        out[:, c0:c1] = (H @ wide(w_lm_store[:, c0:c1])).astype(np.float32)
    return out


# ----------------------------------------------------------------------------
# convenience: a whole workload


def hidden_values(hidden_store: np.ndarray, bf16: bool) -> np.ndarray:
    return bf16_values(hidden_store) if bf16 else np.asarray(hidden_store, np.float64)


def build_all(spec, w: dict, req: dict, requests_subset=None, base=None) -> list:
    """Trees for the requests of a workload (all, or the listed subset).

    `base` overrides the base logits [B, D, V] (the LM-head pipeline passes
    the fp32 logits computed by lm_head_logits).
    """
    bf16 = spec.wdtype == "bf16"
    head = make_head(w, bf16, spec.act_bf16)
    base = req["base"] if base is None else base
    idx = range(spec.B) if requests_subset is None else requests_subset
    out = []
    for b in idx:
        hid = hidden_values(req["hidden"][b], bf16)
        out.append(build_tree(head, base[b], hid, req["root"][b], spec.M, spec.k,
                              spec.N, spec.T, spec.norm))
    return out
