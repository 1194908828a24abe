"""CPU oracle for the tree-attention inputs of a built draft tree.

TEST INFRASTRUCTURE.  Only tests/ (and bench.py's CPU leg, should it ever
need it) may import or run this module; the GPU library never does, and this
module imports nothing from it.

Source: "Riassunto Tecnico: DominoTree", Componenti Core 5 (verification):
the drafted tree is verified with the standard tree attention of
DDTree/SpecInfer, whose causal mask is built from each node's ancestors.

What it computes for one tree (the builder's outputs: node 0 the root, nodes
1..n in pop order, each with a parent of smaller index):
  * mask[i, j] = 1 when node j is node i itself or one of its ancestors
    (the root included), for i, j <= n; rows and columns past n are 0;
  * position[i] = prefix_len + depth[i] for i <= n, -1 past n (the root sits
    at the position right after the committed prefix, a node at depth d d
    places after it);
  * flat[i] = token[i] for 1 <= i <= n, the caller's anchor token (the last
    committed token, which the root stands for) at i = 0, -1 past n.

Readings where the pages say nothing (also in the repository's design notes):
the root is the anchor token and takes part in the mask like any node; the
prefix tokens are not in the mask (every node sees all of them); the mask is
packed 32 columns to a little-endian uint32 word (bit j % 32 of word j // 32).
A tree that breaks the builder's invariants -- n outside [0, cols - 1], a
parent not smaller than its child, a chain not ending at the root with -1, a
depth that is not the chain's length -- is reported as bad; its mask row
holds the nodes the walk reached before the break.
"""
from __future__ import annotations

import numpy as np


def tree_attention_inputs(parents, depths, tokens, n_nodes: int, prefix_len: int = 0,
                          anchor: int = -1):
    """(mask bool [cols, cols], positions int64 [cols], flat int64 [cols], bad bool)."""
    parents = np.asarray(parents, np.int64)
    cols = parents.shape[0]
    mask = np.zeros((cols, cols), dtype=bool)
    positions = np.full(cols, -1, dtype=np.int64)
    flat = np.full(cols, -1, dtype=np.int64)
    bad = not (0 <= n_nodes <= cols - 1)
    n = min(max(int(n_nodes), 0), cols - 1)
    for i in range(n + 1):
        # node i attends to itself and to each node on its path to the root
        j, steps = i, 0
        while True:
            mask[i, j] = True
            p = int(parents[j])
            if p == -1 and j == 0:
                break
            if not (0 <= p < j):
                bad = True
                break
            j, steps = p, steps + 1
        if steps != int(depths[i]):
            bad = True
        positions[i] = prefix_len + int(depths[i])
        flat[i] = anchor if i == 0 else int(tokens[i])
    return mask, positions, flat, bad


def pack_mask(mask: np.ndarray) -> np.ndarray:
    """Bool [rows, cols] -> uint32 [rows, ceil(cols / 32)], bit j % 32 of word j // 32."""
    rows, cols = mask.shape
    words = (cols + 31) // 32
    out = np.zeros((rows, words), dtype=np.uint32)
    for j in range(cols):
        out[:, j // 32] |= mask[:, j].astype(np.uint32) << np.uint32(j % 32)
    return out
