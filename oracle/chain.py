"""CPU oracle for the greedy Domino chain head over the full vocabulary.

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
