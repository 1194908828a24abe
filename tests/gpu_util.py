"""Helpers for the GPU parity tests: run a workload through the C ABI and
compare each request's tree with the oracle's."""
import numpy as np

from oracle import certify, ref
from workloads import synth

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def to_dev(a):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def make_builder(spec, w, max_batch=None, max_m=None, max_k=None, max_n=None):
    import conditional_draft_tree_dominotree_amd as pkg
    tw = {k: to_dev(v) for k, v in w.items()}
    return pkg.TreeBuilder(tw, vocab=spec.V, depths=spec.D, hidden=spec.h, emb_dim=spec.e,
                           state_dim=spec.ds, rank=spec.r, max_batch=max_batch or spec.B,
                           max_top_m=max_m or spec.M, max_top_k=max_k or spec.k,
                           max_budget=max_n or spec.N)


def run(tb, spec, req, base=None, candidates=True, flags=None):
    import conditional_draft_tree_dominotree_amd as pkg
    hidden = to_dev(req["hidden"])
    if base is None and spec.logits != "lmhead":
        base = req["base"]
    root = to_dev(req["root"]) if spec.root_std > 0 else None
    norm = pkg.DT_NORM_FULLV if spec.norm == "fullv" else pkg.DT_NORM_TOPM
    o = tb.outputs(hidden.shape[0], spec.M, spec.N, candidates=candidates, stats=True)
    out = tb.build(hidden, to_dev(base), root, top_m=spec.M, top_k=spec.k, budget=spec.N,
                   temperature=spec.T, norm=norm, flags=flags, out=o)
    tb.sync_status()
    return {k: v.cpu().numpy() for k, v in out.items()}


def oracle_trees(spec, w, req, requests=None, base=None):
    return ref.build_all(spec, w, req, requests_subset=requests, base=base)


def compare(spec, w, req, got, requests=None, base=None, tol=None, logits_computed=False):
    """certify.compare for each listed request; returns the reports.

    Also checks the padding past each request's n_nodes."""
    bf16 = spec.wdtype == "bf16"
    tol = tol if tol is not None else (TOL_BF16 if bf16 else TOL_F32)
    head = ref.make_head(w, bf16, spec.act_bf16)
    idx = list(range(spec.B)) if requests is None else list(requests)
    trees = oracle_trees(spec, w, req, idx, base=base)
    reps = []
    for b, ot in zip(idx, trees):
        hid = ref.hidden_values(req["hidden"][b], bf16)
        other = {k: got[k][b] for k in ("tokens", "parents", "depths", "scores")}
        other["n_nodes"] = int(got["n_nodes"][b])
        extra = {}
        if logits_computed:   # the GPU's candidate sets, checked against the oracle's margins
            extra = dict(cand_other=got["cand_ids"][b], base_rows=base[b])
        reps.append(certify.compare(ot, head, hid, req["root"][b], other, spec.k, spec.T,
                                    spec.norm, spec.N, tol, logits_computed=logits_computed, **extra))
    check_padding(got, spec.N)
    if "stats" in got:
        check_stats(got, spec)
    return reps, trees


def check_stats(got, spec):
    """The builder's per-request stats: at least one step, at most N + 1 (each
    step takes one of the N best nodes), at most 16 expansions per step, and
    every expandable node of the tree (the root, depth < D and index < N)
    expanded."""
    for b in range(got["n_nodes"].shape[0]):
        steps, expanded = (int(x) for x in got["stats"][b])
        n = int(got["n_nodes"][b])
        need = sum(1 for i in range(n + 1) if got["depths"][b, i] < spec.D and i < spec.N)
        assert 1 <= steps <= spec.N + 1, (b, steps)
        assert need <= expanded <= 16 * steps, (b, expanded, need, steps)


def check_padding(got, N):
    """Slots past n_nodes: token -1, parent -1, depth -1, score -inf."""
    for b in range(got["n_nodes"].shape[0]):
        n = int(got["n_nodes"][b])
        assert 0 <= n <= N, (b, n)
        for key, pad in (("tokens", -1), ("parents", -1), ("depths", -1)):
            assert np.all(got[key][b, n + 1:N + 1] == pad), (b, key)
        assert np.all(np.isneginf(got["scores"][b, n + 1:N + 1])), (b, "scores")


def assert_parity(reps, ids=None):
    """Every tree passes the certificate and is exact unless the oracle itself
    met a decision within the tolerance (then only a difference excused by a
    near tie at the decision that produced it is allowed)."""
    ids = list(range(len(reps))) if ids is None else list(ids)
    for b, r in zip(ids, reps):
        assert r.ok, (b, r)
        assert r.exact or not r.must_be_exact, (b, r)


def check_candidates(spec, trees, got, requests, exact=True):
    for b, ot in zip(requests, trees):
        for d, dep in enumerate(ot.depths_info):
            ids = got["cand_ids"][b, d]
            if exact:
                np.testing.assert_array_equal(ids, dep.cand, err_msg=f"request {b} depth {d}")
                np.testing.assert_array_equal(got["cand_logits"][b, d], dep.base.astype(np.float32))
            lse = got["lse"][b, d]
            assert abs(lse - dep.lse) <= 2e-5 * max(1.0, abs(dep.lse)), (b, d, lse, dep.lse)


def summarize(reps):
    n_exact = sum(r.exact for r in reps)
    ties = [r.near_tie for r in reps if not r.exact]
    worst = max((r.max_dscore for r in reps), default=0.0)
    must = sum(r.must_be_exact for r in reps)
    cen = {}
    for r in reps:
        for key, v in r.census.items():
            cen[key] = cen.get(key, 0) + v
    swaps = sum(r.topm_swaps for r in reps)
    return (f"{n_exact}/{len(reps)} exact, near-ties {ties}, top-M swaps {swaps}, max|dscore| {worst:.3e}; "
            f"census: {must}/{len(reps)} trees with no oracle decision within tol, "
            f"decisions within tol {cen}")
