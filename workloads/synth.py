"""Seeded synthetic inputs for the conditional draft-tree builder.

This module draws random numbers and stores them; it computes no step of the
tree-building method. Both the CPU oracle (test infrastructure) and the GPU
library consume what it returns, so it is the one module they share.

Workloads (shapes and distributions follow the Domino / DominoTree pages:
Domino head hyper-parameters -- block 16, GRU state 1024, correction rank 256
-- from the Domino summary, "reproduction" section; the Qwen3-4B/8B hidden
sizes and the 151936-token vocabulary are the targets those pages evaluate):

  tiny     fp32, V=1024, 7 depths, h=e=128, d_s=64, r=32, M=8, k=4, N=32, T=1
  q4b_b1   bf16, Qwen3-4B shape (h=e=2560), batch 1, M=32, k=8, N=64, T=1
  q8b_b1   bf16, Qwen3-8B shape (h=e=4096), batch 1, M=32, k=8, N=128, T=1
  q8b_b32  as q8b_b1 with 32 independent requests, T=0.5
  q8b_lm   32 requests from RMS-normalised hidden states through a bf16 LM
           head [4096, 151936]; M=64, k=8, N=256, T=1

Distribution conventions: a "fan-in" draw has variance 1/fan_in; other
normal draws are given by their standard deviation.  bf16 tensors are drawn
in fp32 and rounded to nearest-even; they are returned as uint16 bit patterns.

Every tensor (or row block of one) has its own seed,
SeedSequence([ROOT, group, tensor_id, block]), so any part can be regenerated
alone and the draws never depend on which other tensors were generated.
"""
from __future__ import annotations

import dataclasses
import functools
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

ROOT_SEED = 0x0D0A1E  # fixed root of every seed in this module

# tensor ids inside a seed group
_T_EMB, _T_WIH, _T_WHH, _T_W1, _T_W2, _T_WLM, _T_BIH, _T_BHH = range(8)
_T_LOGITS, _T_HIDDEN, _T_BOOST, _T_ROOT = 16, 17, 18, 19


@dataclass(frozen=True)
class Spec:
    name: str
    V: int          # vocabulary
    D: int          # draft depths (block size minus one)
    h: int          # backbone hidden size (H_d rows, W1_H rows)
    e: int          # embedding size (GRU input)
    ds: int         # GRU state size
    r: int          # correction rank
    M: int          # per-depth candidates
    k: int          # children per expansion
    N: int          # node budget (non-root)
    T: float        # temperature
    B: int          # requests
    wdtype: str     # "f32" or "bf16" (weights, embeddings, hidden states)
    logits: str     # "boost" | "zipf" | "lmhead"
    wgroup: int     # seed group of the shared weights
    group: int      # seed group of the per-request tensors
    norm: str = "topm"        # "topm" | "fullv"
    emb_std: float = 0.02     # embedding std (tiny uses 1.0)
    biases: bool = False      # draw GRU biases (tests only; the workloads use none)
    root_std: float = 0.0     # std of a random root state (0 = zeros)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)

    @property
    def act_bf16(self) -> bool:
        return self.wdtype == "bf16"


SPECS = {
    "tiny": Spec("tiny", V=1024, D=7, h=128, e=128, ds=64, r=32, M=8, k=4, N=32,
                 T=1.0, B=1, wdtype="f32", logits="boost", wgroup=0, group=0,
                 emb_std=1.0),
    "q4b_b1": Spec("q4b_b1", V=151936, D=15, h=2560, e=2560, ds=1024, r=256, M=32,
                   k=8, N=64, T=1.0, B=1, wdtype="bf16", logits="zipf", wgroup=1,
                   group=1),
    "q8b_b1": Spec("q8b_b1", V=151936, D=15, h=4096, e=4096, ds=1024, r=256, M=32,
                   k=8, N=128, T=1.0, B=1, wdtype="bf16", logits="zipf", wgroup=2,
                   group=2),
    "q8b_b32": Spec("q8b_b32", V=151936, D=15, h=4096, e=4096, ds=1024, r=256, M=32,
                    k=8, N=128, T=0.5, B=32, wdtype="bf16", logits="zipf", wgroup=2,
                    group=3),
    "q8b_lm": Spec("q8b_lm", V=151936, D=15, h=4096, e=4096, ds=1024, r=256, M=64,
                   k=8, N=256, T=1.0, B=32, wdtype="bf16", logits="lmhead", wgroup=2,
                   group=4),
}
ORDER = ["tiny", "q4b_b1", "q8b_b1", "q8b_b32", "q8b_lm"]


def small(name="small", *, V=6, D=3, h=8, e=8, ds=4, r=4, M=None, k=None, N=8,
          T=1.0, B=1, wdtype="f32", logits="boost", group=100, **kw) -> Spec:
    """A small fp32 (or bf16) instance for brute force and edge cases."""
    M = V if M is None else M
    k = M if k is None else k
    return Spec(name, V=V, D=D, h=h, e=e, ds=ds, r=r, M=M, k=k, N=N, T=T, B=B,
                wdtype=wdtype, logits=logits, wgroup=group, group=group,
                emb_std=kw.pop("emb_std", 1.0), **kw)


# ----------------------------------------------------------------------------
# drawing helpers


def _rng(group: int, tid: int, block: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([ROOT_SEED, group, tid, block]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen stored bf16 bit patterns to the fp32 values they denote."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x32: np.ndarray, wdtype: str) -> np.ndarray:
    return bf16_bits(x32) if wdtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _normal_rows(rows: int, cols: int, std: float, group: int, tid: int,
                 wdtype: str, block_rows: int = 2048) -> np.ndarray:
    """[rows, cols] normal(0, std^2) draws, row blocks seeded independently."""
    out = np.empty((rows, cols), np.uint16 if wdtype == "bf16" else np.float32)

    def fill(b0):
        b1 = min(rows, b0 + block_rows)
        x = _rng(group, tid, b0 // block_rows).standard_normal((b1 - b0, cols),
                                                              dtype=np.float32)
        x *= np.float32(std)
        out[b0:b1] = _store(x, wdtype)

    _parallel(fill, range(0, rows, block_rows))
    return out


def _parallel(fn, items):
    items = list(items)
    if len(items) <= 1:
        for it in items:
            fn(it)
        return
    n = max(1, min(16, len(os.sched_getaffinity(0)), len(items)))
    with ThreadPoolExecutor(n) as ex:
        list(ex.map(fn, items))


# ----------------------------------------------------------------------------
# weights (shared by every request of a workload)


@functools.lru_cache(maxsize=2)
def weights(spec: Spec) -> dict:
    """Domino head weights and the embedding table.

    emb [V, e]; w_ih [3 d_s, e] and w_hh [3 d_s, d_s] with gate row blocks in
    (reset, update, new) order; w1 [h + d_s, r] acting as x @ w1 on the
    concatenation [H_d; S]; w2 [r, V]; w_lm [h, V] for the LM-head workload.
    b_ih / b_hh are fp32 [3 d_s] or None.
    """
    g, wd = spec.wgroup, spec.wdtype
    w = {
        "emb": _normal_rows(spec.V, spec.e, spec.emb_std, g, _T_EMB, wd),
        "w_ih": _normal_rows(3 * spec.ds, spec.e, spec.e ** -0.5, g, _T_WIH, wd),
        "w_hh": _normal_rows(3 * spec.ds, spec.ds, spec.ds ** -0.5, g, _T_WHH, wd),
        "w1": _normal_rows(spec.h + spec.ds, spec.r, (spec.h + spec.ds) ** -0.5, g,
                           _T_W1, wd),
        "w2": _normal_rows(spec.r, spec.V, spec.r ** -0.5, g, _T_W2, wd, block_rows=16),
        "b_ih": None,
        "b_hh": None,
        "w_lm": None,
    }
    if spec.biases:
        w["b_ih"] = _rng(g, _T_BIH).standard_normal(3 * spec.ds, dtype=np.float32) * 0.5
        w["b_hh"] = _rng(g, _T_BHH).standard_normal(3 * spec.ds, dtype=np.float32) * 0.5
    if spec.logits == "lmhead":
        w["w_lm"] = _normal_rows(spec.h, spec.V, spec.h ** -0.5, g, _T_WLM, wd,
                                 block_rows=256)
    return w


# ----------------------------------------------------------------------------
# per-request inputs


def _zipf_row(V: int, rng: np.random.Generator) -> np.ndarray:
    """Zipf-shaped logits: -1.1 ln(rank) + N(0, 0.5^2), ranks on a random permutation."""
    ranks = np.arange(1, V + 1, dtype=np.float64)
    val = (-1.1 * np.log(ranks)).astype(np.float32)
    val += rng.standard_normal(V, dtype=np.float32) * np.float32(0.5)
    perm = rng.permutation(V)
    row = np.empty(V, np.float32)
    row[perm] = val
    return row


def _boost_row(V: int, rng: np.random.Generator) -> np.ndarray:
    """N(0,1)*2 logits with 1-3 distinct uniformly drawn ids boosted by +4."""
    row = rng.standard_normal(V, dtype=np.float32) * np.float32(2.0)
    cnt = int(rng.integers(1, 4))
    ids = rng.choice(V, size=cnt, replace=False)
    row[ids] += np.float32(4.0)
    return row


@functools.lru_cache(maxsize=2)
def requests(spec: Spec) -> dict:
    """Per-request tensors.

    base  [B, D, V] fp32 base logits (None for the LM-head workload)
    hidden [B, D, h] backbone hidden states (bf16 bits or fp32)
    root  [B, d_s] fp32 root GRU state
    """
    g = spec.group
    B, D, V = spec.B, spec.D, spec.V
    base = None
    if spec.logits in ("zipf", "boost"):
        base = np.empty((B, D, V), np.float32)

        def fill(i):
            rng = _rng(g, _T_LOGITS, i)
            row = _zipf_row(V, rng) if spec.logits == "zipf" else _boost_row(V, rng)
            base[i // D, i % D] = row

        _parallel(fill, range(B * D))
    hid32 = np.empty((B, D, spec.h), np.float32)
    for b in range(B):
        hid32[b] = _rng(g, _T_HIDDEN, b).standard_normal((D, spec.h), dtype=np.float32)
    if spec.logits == "lmhead":
        # the drafter's final RMS normalisation (no gain)
        ms = np.mean(hid32.astype(np.float64) ** 2, axis=-1, keepdims=True)
        hid32 = (hid32 / np.sqrt(ms + 1e-6)).astype(np.float32)
    hidden = _store(hid32, spec.wdtype)
    root = np.zeros((B, spec.ds), np.float32)
    if spec.root_std > 0:
        for b in range(B):
            root[b] = _rng(g, _T_ROOT, b).standard_normal(spec.ds, dtype=np.float32) \
                * np.float32(spec.root_std)
    return {"base": base, "hidden": hidden, "root": root}


def workload(name_or_spec) -> tuple[Spec, dict, dict]:
    spec = SPECS[name_or_spec] if isinstance(name_or_spec, str) else name_or_spec
    return spec, weights(spec), requests(spec)
