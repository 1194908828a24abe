"""GPU parity at the full workload sizes (Qwen3-4B / Qwen3-8B shapes).

The oracle rebuilds a sample of requests one by one; every request of the
batch is checked for the properties that hold at any size (exact candidates,
valid tree structure, full budget, non-increasing scores in pop order).
"""
import numpy as np
import pytest

from tests import gpu_util as gu
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def q8b_builder(dev):
    # the LM-head workload draws the same Qwen3-8B-shaped head weights (same
    # seed group) plus W_lm, so one handle serves every q8b workload
    spec, w, _ = synth.workload("q8b_lm")
    tb = gu.make_builder(spec, w, max_batch=32, max_m=64, max_k=8, max_n=256)
    yield tb
    tb.close()


def _top_m_fast(row, M):
    # (value desc, id asc) over the whole row, via a partition then an exact sort
    kth = np.partition(row, row.size - M)[row.size - M]
    idx = np.nonzero(row >= kth)[0]
    order = np.lexsort((idx, -row[idx].astype(np.float64)))
    return idx[order][:M]


def _check_structure(spec, got):
    for b in range(spec.B):
        n = int(got["n_nodes"][b])
        assert n == spec.N, (b, n)
        par, dep, sc = got["parents"][b], got["depths"][b], got["scores"][b]
        assert par[0] == -1 and dep[0] == 0 and sc[0] == 0
        for i in range(1, n + 1):
            assert 0 <= par[i] < i and dep[i] == dep[par[i]] + 1 <= spec.D
        assert np.all(np.diff(sc[1:n + 1]) <= 1e-6)


def _full_case(spec, w, req, tb, sample):
    got = gu.run(tb, spec, req)
    _check_structure(spec, got)
    for b in range(spec.B):
        for d in range(spec.D):
            np.testing.assert_array_equal(got["cand_ids"][b, d], _top_m_fast(req["base"][b, d], spec.M),
                                          err_msg=f"request {b} depth {d}")
    reps, trees = gu.compare(spec, w, req, got, requests=sample)
    gu.check_candidates(spec, trees, got, sample)
    print(spec.name, gu.summarize(reps))
    gu.assert_parity(reps, sample)
    return got, reps


def test_q4b_b1(dev):
    spec, w, req = synth.workload("q4b_b1")
    tb = gu.make_builder(spec, w)
    _full_case(spec, w, req, tb, [0])
    tb.close()


def test_q8b_b1(dev, q8b_builder):
    spec, w, req = synth.workload("q8b_b1")
    _full_case(spec, w, req, q8b_builder, [0])


def test_q8b_b32(dev, q8b_builder):
    # every request of the batch against the oracle (about 6 s of CPU)
    spec, w, req = synth.workload("q8b_b32")
    _full_case(spec, w, req, q8b_builder, list(range(spec.B)))


def test_q8b_b32_one_half(dev, q8b_builder):
    # the register workers serving the whole batch at each step (the default
    # at 32 requests serves it in two halves)
    q8b_builder.set_schedule(halves=1)
    try:
        spec, w, req = synth.workload("q8b_b32")
        _full_case(spec, w, req, q8b_builder, [0, 17, 31])
    finally:
        q8b_builder.set_schedule()


def test_q8b_b32_lds_workers(dev, q8b_builder):
    # the workers that stage operands in LDS (the schedule for d_s other than
    # 1024) at the full shape, on the same handle
    q8b_builder.set_schedule(lds_workers=1)
    try:
        spec, w, req = synth.workload("q8b_b32")
        _full_case(spec, w, req, q8b_builder, [0, 31])
    finally:
        q8b_builder.set_schedule()


def test_q8b_b32_fma_correction(dev, q8b_builder):
    # the expansions' correction dL with vector FMAs instead of the matrix
    # cores, at the full shape
    q8b_builder.set_schedule(dl=1)
    try:
        spec, w, req = synth.workload("q8b_b32")
        _full_case(spec, w, req, q8b_builder, [3, 30])
    finally:
        q8b_builder.set_schedule()


def test_q8b_b32_device_wide_exchange_same_trees(dev, q8b_builder):
    # the column groups' state exchange through their XCD's L2 (the default
    # where a group runs on one XCD) and device-wide move the same values in
    # the same order: the trees are the same bit for bit
    spec, w, req = synth.workload("q8b_b32")
    local = gu.run(q8b_builder, spec, req)
    q8b_builder.set_schedule(exchange=1)
    try:
        device = gu.run(q8b_builder, spec, req)
    finally:
        q8b_builder.set_schedule()
    for key in ("tokens", "parents", "depths", "scores", "n_nodes"):
        np.testing.assert_array_equal(local[key], device[key], err_msg=key)
    reps, _ = gu.compare(spec, w, req, device, requests=[0, 31])
    gu.assert_parity(reps, [0, 31])


def test_q8b_b32_cooperative_launch_same_trees(dev, q8b_builder):
    # the cooperative launch (schedule launch = 2) runs the same kernel as
    # the default plain launch: the same trees bit for bit
    spec, w, req = synth.workload("q8b_b32")
    plain = gu.run(q8b_builder, spec, req)
    q8b_builder.set_schedule(launch=2)
    try:
        coop = gu.run(q8b_builder, spec, req)
    finally:
        q8b_builder.set_schedule()
    for key in ("tokens", "parents", "depths", "scores", "n_nodes"):
        np.testing.assert_array_equal(plain[key], coop[key], err_msg=key)


def test_q8b_b32_plain_launch_beside_another_streams_work(dev, q8b_builder):
    # the default plain launch while another stream's matrix products hold
    # the compute units: builder blocks that wait for a unit start once the
    # products' blocks retire, well inside the bounded waits, and the trees
    # are those of the idle GPU
    import torch

    import conditional_draft_tree_dominotree_amd as pkg
    spec, w, req = synth.workload("q8b_b32")
    want = gu.run(q8b_builder, spec, req)
    hidden, base = gu.to_dev(req["hidden"]), gu.to_dev(req["base"])
    out = q8b_builder.outputs(spec.B, spec.M, spec.N)
    x = torch.randn(4096, 4096, device=dev)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for _ in range(6):
            x = torch.tanh(x @ x * 1e-3)
    q8b_builder.build(hidden, base, None, top_m=spec.M, top_k=spec.k, budget=spec.N, temperature=spec.T,
                      flags=pkg.DT_ACT_BF16, out=out)
    torch.cuda.synchronize()
    q8b_builder.sync_status()
    for key in ("tokens", "parents", "depths", "scores", "n_nodes"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), want[key], err_msg=key)


def test_q8b_b32_fullv_and_smaller_batch_reuse_handle(dev, q8b_builder):
    # the same handle serves a smaller batch and the full-vocabulary normaliser
    spec, w, req = synth.workload("q8b_b32")
    small = spec.replace(B=5, norm="fullv", N=96)
    req5 = {k: (v[:5] if v is not None else None) for k, v in req.items()}
    _full_case(small, w, req5, q8b_builder, [0, 4])


def test_q8b_lm_pipeline(dev, q8b_builder):
    # every request of the LM-head pipeline: the GPU's base logits element by
    # element, its candidates, and its trees against the oracle's (which
    # computes the base logits itself, in float64, rounded to fp32)
    from oracle import ref
    spec, w, req = synth.workload("q8b_lm")
    B, D, V, K = spec.B, spec.D, spec.V, spec.h
    o = q8b_builder.outputs(B, spec.M, spec.N, candidates=True, stats=True, logits=True)
    import conditional_draft_tree_dominotree_amd as pkg
    q8b_builder.build(gu.to_dev(req["hidden"]), None, None, top_m=spec.M, top_k=spec.k, budget=spec.N,
                      temperature=spec.T, flags=pkg.DT_ACT_BF16, out=o)
    q8b_builder.sync_status()
    got = {k: v.cpu().numpy() for k, v in o.items()}
    _check_structure(spec, got)
    rows = req["hidden"].reshape(B * D, K)
    base = ref.lm_head_logits(rows, w["w_lm"], True).reshape(B, D, V)
    # fp32 accumulation of K exact bf16 products in any order errs by at most
    # gamma_K sum|h_i w_i| <= gamma_K |h| |w| (Cauchy-Schwarz); the oracle's
    # fp32 rounding adds half an ulp
    hn = np.linalg.norm(ref.bf16_values(rows), axis=1)
    wn = np.empty(V)
    for c0 in range(0, V, 8192):
        wc = ref.bf16_values(w["w_lm"][:, c0:c0 + 8192])
        wn[c0:c0 + 8192] = np.sqrt(np.sum(wc * wc, axis=0))
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    err = np.abs(got["logits"].astype(np.float64) - base).reshape(B * D, V)
    bound = gamma * hn[:, None] * wn[None, :] + np.spacing(np.abs(base).astype(np.float32)).reshape(B * D, V)
    worst = float(err.max())
    print(f"{spec.name} logits: max |gpu - oracle| {worst:.3e} over {err.size} elements, "
          f"bound at least {float(bound.min()):.3e}")
    assert np.all(err <= bound)
    assert worst <= 1e-4
    margins = []
    # candidate sets may differ only at a top-M boundary within 1e-4 of the
    # oracle's logits (checked by the comparison, which then compares with the
    # oracle's tree on the GPU's sets)
    reps, trees = gu.compare(spec, w, req, got, base=base, logits_computed=True)
    for b, t in enumerate(trees):
        for d, dep in enumerate(t.depths_info):
            margins.append(dep.margin)
            lse = got["lse"][b, d]
            assert abs(lse - dep.lse) <= 1e-4 * max(1.0, abs(dep.lse)), (b, d, lse, dep.lse)
            # the candidates' logits are the GPU's own logits at those ids, in
            # its own (value desc, id asc) order
            ids, vals = got["cand_ids"][b, d], got["cand_logits"][b, d]
            np.testing.assert_array_equal(vals, got["logits"][b, d, ids])
            assert all((vals[i] > vals[i + 1]) or (vals[i] == vals[i + 1] and ids[i] < ids[i + 1])
                       for i in range(len(ids) - 1)), (b, d)
    print(spec.name, gu.summarize(reps), f"smallest top-M margin {min(margins):.3e}")
    gu.assert_parity(reps)


def test_q8b_b32_marginal(dev, q8b_builder):
    import conditional_draft_tree_dominotree_amd as pkg
    spec, w, req = synth.workload("q8b_b32")
    got = gu.run(q8b_builder, spec, req, flags=pkg.DT_ACT_BF16 | pkg.DT_MARGINAL)
    _check_structure(spec, got)
    w0 = dict(w)
    w0["w2"] = np.zeros_like(w["w2"])
    reps, _ = gu.compare(spec, w0, req, got, requests=[0, 13, 31])
    print(spec.name, "marginal", gu.summarize(reps))
    gu.assert_parity(reps, [0, 13, 31])


def test_q8b_b32_repeated_builds_bitwise(dev, q8b_builder):
    # 200 back-to-back builds of the full batch (two halves per step): every
    # decision is taken in a fixed order, so each build must return the first
    # build's trees bit for bit; a race in the exchange between the halves
    # would show up as a differing tree
    import torch
    spec, w, req = synth.workload("q8b_b32")
    first = gu.run(q8b_builder, spec, req)
    hidden, base = gu.to_dev(req["hidden"]), gu.to_dev(req["base"])
    import conditional_draft_tree_dominotree_amd as pkg
    out = q8b_builder.outputs(spec.B, spec.M, spec.N)
    for i in range(200):
        q8b_builder.build(hidden, base, None, top_m=spec.M, top_k=spec.k, budget=spec.N,
                          temperature=spec.T, norm=pkg.DT_NORM_TOPM, flags=pkg.DT_ACT_BF16, out=out)
        if i % 50 == 49:
            torch.cuda.synchronize()
            q8b_builder.sync_status()
            for key in ("tokens", "parents", "depths", "scores", "n_nodes"):
                np.testing.assert_array_equal(out[key].cpu().numpy(), first[key], err_msg=f"{key} build {i}")
