"""CPU oracle for the Domino chain head over the full vocabulary: greedy and
sampled.

TEST INFRASTRUCTURE.  Only tests/ and bench.py's CPU leg may import or run
this module; the GPU library never does, and this module imports nothing
from it.

Source: "Domino：在投机解码中将因果建模与自回归草稿解耦", sections 核心方法 and
方法步骤详情: the Domino head corrects the block-parallel base logits of each
draft position i with dL_i = W2 SiLU(W1 [H_i; S_{i-1}]), where the causal
state S is a GRU over the embeddings of the tokens drafted before position i;
at inference the state is advanced from the previously drafted token, one
position at a time (the loop the page's fused kernel runs).  The chain here
is the greedy one: each position takes the token with the largest corrected
logit base + dL over the whole vocabulary.

Readings (also in the repository's design notes): the state before the first
position is the caller's root state (zeros by default), as for the tree
builder's root; ties go to the lowest token id; the temperature does not
change a greedy pick and is not an input; bf16 weights follow the tree
builder's rounding points (the state rounded to bf16 only as a matrix
operand, dL from fp32 SiLU outputs and bf16 W2).

The sampled chain draws each position's token from the refined logits, as
the Domino page's inference step does, at temperature T: from
softmax((base + dL) / T).  The draw is the Gumbel-max rule (the argmax of
the tempered logits plus independent standard Gumbel noise is distributed as
that softmax), with the noise derived from a counter-based generator,
Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
easy as 1, 2, 3", SC 2011), so that a seed fixes every draw:
  word w = Philox4x32-10(counter (floor(v / 4), d, b, 0), key (seed mod 2^32,
           floor(seed / 2^32)))[v mod 4] for token v, position d (0-based),
  request row b;
  u = (floor(w / 2^9) + 1/2) / 2^23, in (0, 1), exact in fp32;
  g = -ln(-ln u).
Readings: the noise layout above is this library's definition (the pages
name no generator); T > 0 (T = 0 is the greedy chain).
"""
from __future__ import annotations

import numpy as np

from oracle import ref


def greedy_chain(head: ref.Head, base: np.ndarray, hidden: np.ndarray, root: np.ndarray):
    """tokens [D], corrected logits of the picks [D], pick margins [D] (the
    gap to the runner-up, for the near-tie census)."""
    D, V = base.shape
    w2 = head.w2_cols(np.arange(V))          # [r, V] widened once
    ids = np.arange(V)
    s = np.asarray(root, np.float64)
    tokens, logits, margins = [], [], []
    for d in range(D):
        u = np.concatenate([hidden[d], ref.operand(head, s)]) @ head.w1
        z = base[d].astype(np.float64) + w2.T @ ref.silu(u)
        order = ref.rank_desc(z, ids)
        x = int(order[0])
        tokens.append(x)
        logits.append(float(z[x]))
        margins.append(float(z[x] - z[order[1]]) if V > 1 else float("inf"))
        if d + 1 < D:
            s = ref.gru_step(head, s, head.emb(x))
    return np.array(tokens), np.array(logits), np.array(margins)


def fold_state(head: ref.Head, prev: np.ndarray, tokens) -> np.ndarray:
    """The causal state after the committed tokens: S <- GRU(S, E[t]) for each
    token in order, from `prev` [Domino, Method: the state is a GRU over the
    embeddings of the tokens before the position]."""
    s = np.asarray(prev, np.float64)
    for t in tokens:
        s = ref.gru_step(head, s, head.emb(int(t)))
    return s


# ---- Philox4x32-10 (Salmon et al., SC 2011) --------------------------------
PHILOX_M = (0xD2511F53, 0xCD9E8D57)   # round multipliers
PHILOX_W = (0x9E3779B9, 0xBB67AE85)   # key schedule increments (Weyl sequence)
_M32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """ctr [..., 4] and key [..., 2] (uint32 values) -> [..., 4] uint32.
    Ten rounds; round i uses the key plus i times the Weyl increments.  A
    round multiplies words 0 and 2 by the two multipliers and forms
    (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))."""
    c = [np.asarray(ctr, np.uint64)[..., i] & _M32 for i in range(4)]
    k0 = np.asarray(key, np.uint64)[..., 0] & _M32
    k1 = np.asarray(key, np.uint64)[..., 1] & _M32
    m0, m1 = np.uint64(PHILOX_M[0]), np.uint64(PHILOX_M[1])
    for i in range(10):
        if i:
            k0 = (k0 + np.uint64(PHILOX_W[0])) & _M32
            k1 = (k1 + np.uint64(PHILOX_W[1])) & _M32
        p0 = m0 * c[0]  # < 2^64: no wrap in uint64
        p1 = m1 * c[2]
        c = [((p1 >> np.uint64(32)) ^ c[1] ^ k0) & _M32, p1 & _M32,
             ((p0 >> np.uint64(32)) ^ c[3] ^ k1) & _M32, p0 & _M32]
    return np.stack(c, -1).astype(np.uint32)


def chain_words(seed: int, b: int, d: int, V: int) -> np.ndarray:
    """The generator's word for every token 0..V-1 of request row b at
    position d (the layout in the module docstring)."""
    v4 = np.arange((V + 3) // 4, dtype=np.uint64)
    ctr = np.stack([v4, np.full_like(v4, d), np.full_like(v4, b), np.zeros_like(v4)], -1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], np.uint64)
    return philox4x32_10(ctr, np.broadcast_to(key, ctr.shape[:-1] + (2,))).reshape(-1)[:V]


def uniforms(words: np.ndarray) -> np.ndarray:
    """u = (floor(w / 2^9) + 1/2) / 2^23 in float64 (each value is an odd
    multiple of 2^-24, so fp32 holds it exactly)."""
    return ((np.asarray(words, np.uint64) >> np.uint64(9)).astype(np.float64) + 0.5) / 2.0 ** 23


def gumbel(u: np.ndarray) -> np.ndarray:
    """Standard Gumbel variates from uniforms: g = -ln(-ln u)."""
    return -np.log(-np.log(u))


def sampled_chain(head: ref.Head, base: np.ndarray, hidden: np.ndarray, root: np.ndarray, temperature: float,
                  seed: int, row: int):
    """The chain with each token drawn from softmax((base + dL) / T) by the
    Gumbel-max rule: x_d = argmax_v ((base + dL)_v / T + g_v), ties to the
    lowest id, g from the seeded generator at (row, d).  Returns tokens [D],
    the corrected logits base + dL of the picks [D] and the margins of the
    perturbed scores over their runners-up [D] (the near-tie census)."""
    assert temperature > 0
    D, V = base.shape
    w2 = head.w2_cols(np.arange(V))
    ids = np.arange(V)
    s = np.asarray(root, np.float64)
    tokens, logits, margins = [], [], []
    for d in range(D):
        u = np.concatenate([hidden[d], ref.operand(head, s)]) @ head.w1
        z = base[d].astype(np.float64) + w2.T @ ref.silu(u)
        score = z / temperature + gumbel(uniforms(chain_words(seed, row, d, V)))
        order = ref.rank_desc(score, ids)
        x = int(order[0])
        tokens.append(x)
        logits.append(float(z[x]))
        margins.append(float(score[x] - score[order[1]]) if V > 1 else float("inf"))
        if d + 1 < D:
            s = ref.gru_step(head, s, head.emb(x))
    return np.array(tokens), np.array(logits), np.array(margins)
