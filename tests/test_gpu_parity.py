"""GPU parity: the HIP path (through the C ABI) against the CPU oracle."""
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
    import conditional_draft_tree_dominotree_amd as pkg
    pkg.load_library()
    return torch.device("cuda:0")


def _assert_ok(reps):
    gu.assert_parity(reps)


def test_tiny_workload(dev):
    spec, w, req = synth.workload("tiny")
    tb = gu.make_builder(spec, w)
    got = gu.run(tb, spec, req)
    reps, trees = gu.compare(spec, w, req, got)
    print(gu.summarize(reps))
    _assert_ok(reps)
    assert reps[0].exact
    gu.check_candidates(spec, trees, got, [0])
    tb.close()


SMALL = [
    # name, kwargs
    ("base", dict(V=1000, D=5, h=32, e=24, ds=64, r=32, M=8, k=3, N=30)),
    ("ragged_two_chunks", dict(V=8195, D=4, h=16, e=16, ds=32, r=16, M=12, k=4, N=25)),
    ("batch3_fullv_T05", dict(V=3000, D=6, h=32, e=32, ds=64, r=48, M=16, k=4, N=40, B=3,
                              norm="fullv", T=0.5)),
    ("biases_root", dict(V=500, D=4, h=8, e=8, ds=12, r=8, M=6, k=2, N=20, biases=True,
                         root_std=0.7)),
    ("chain_k1", dict(V=700, D=6, h=16, e=16, ds=32, r=16, M=8, k=1, N=40)),
    ("n1", dict(V=700, D=6, h=16, e=16, ds=32, r=16, M=8, k=4, N=1)),
    ("m1", dict(V=300, D=5, h=16, e=16, ds=32, r=16, M=1, k=1, N=9)),
    ("m_eq_v", dict(V=6, D=3, h=8, e=8, ds=4, r=4, M=6, k=6, N=100)),
    ("m64_k8_b8", dict(V=20000, D=7, h=64, e=64, ds=128, r=64, M=64, k=8, N=120, B=8)),
    ("deep_d31", dict(V=400, D=31, h=16, e=16, ds=32, r=16, M=4, k=2, N=80)),
    ("max_budget_n1024", dict(V=1500, D=12, h=16, e=16, ds=32, r=16, M=16, k=4, N=1024, B=2)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_fp32(dev, name, kw):
    spec = synth.small(name, group=300 + len(name), **kw)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    got = gu.run(tb, spec, req)
    reps, trees = gu.compare(spec, w, req, got)
    print(name, gu.summarize(reps))
    _assert_ok(reps)
    gu.check_candidates(spec, trees, got, range(spec.B))
    tb.close()


# d_s = 1024 runs the register-resident workers (one or two tiles per wave),
# other sizes the workers that stage operands in LDS
@pytest.mark.parametrize("B,M,k,N,ds", [(1, 16, 4, 40, 128), (5, 32, 8, 64, 128), (32, 16, 4, 50, 128),
                                        (1, 16, 4, 40, 1024), (3, 8, 3, 30, 1024), (32, 8, 4, 24, 1024)])
def test_small_bf16(dev, B, M, k, N, ds):
    spec = synth.small(f"bf16_{B}_{M}_{ds}", V=5000, D=8, h=64, e=96, ds=ds, r=64, M=M, k=k, N=N,
                       B=B, wdtype="bf16", group=400 + B + (0 if ds == 128 else ds), emb_std=0.5)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    got = gu.run(tb, spec, req)
    reps, trees = gu.compare(spec, w, req, got)
    print(gu.summarize(reps))
    _assert_ok(reps)
    gu.check_candidates(spec, trees, got, range(spec.B))
    tb.close()


# the correction dL of an expansion: on the matrix cores (bf16, r a multiple of
# 32; M = 40 leaves a ragged 16-candidate block and takes a wave per node in
# the softmax) and with vector FMAs (r = 48; or forced by the schedule, which
# takes the quad-per-four-candidates form at r = 64)
@pytest.mark.parametrize("r,M,dl", [(96, 40, 0), (32, 16, 0), (48, 16, 0), (64, 16, 1), (64, 40, 1)])
def test_bf16_correction_paths(dev, r, M, dl):
    spec = synth.small(f"bf16_dl_{r}_{M}_{dl}", V=4000, D=7, h=64, e=96, ds=1024, r=r, M=M, k=4, N=48,
                       B=6, wdtype="bf16", group=1700 + r + M + dl, emb_std=0.5)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    tb.set_schedule(dl=dl)
    got = gu.run(tb, spec, req)
    reps, trees = gu.compare(spec, w, req, got)
    print(f"r={r} M={M} dl={dl}", gu.summarize(reps))
    _assert_ok(reps)
    gu.check_candidates(spec, trees, got, range(spec.B))
    tb.close()


def test_bf16_register_workers_with_root_and_biases(dev):
    # a given root state: the workers compute step 0's products (with zero
    # roots the controllers set them up and the workers start at step 1)
    spec = synth.small("bf16_root", V=3000, D=6, h=64, e=96, ds=1024, r=64, M=8, k=3, N=30, B=4,
                       wdtype="bf16", group=977, emb_std=0.5, biases=True, root_std=0.7)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    got = gu.run(tb, spec, req)
    reps, trees = gu.compare(spec, w, req, got)
    print(gu.summarize(reps))
    _assert_ok(reps)
    gu.check_candidates(spec, trees, got, range(spec.B))
    tb.close()


def test_candidates_with_ties_zero_and_inf(dev):
    spec = synth.small("ties", V=20000, D=4, h=16, e=16, ds=32, r=16, M=40, k=4, N=20,
                       group=500)
    spec, w, req = synth.workload(spec)
    base = req["base"].copy()
    rng = np.random.default_rng(0)
    base[0, 0, rng.choice(20000, 300, replace=False)] = 2.5         # many ties at the top
    base[0, 1, :] = np.float32(-0.0)
    base[0, 1, rng.choice(20000, 50, replace=False)] = np.float32(0.0)  # +0 and -0 tie
    base[0, 2, :] = -np.inf
    base[0, 2, [5, 19999, 8191, 8192]] = [1.0, 1.0, 0.5, 0.5]        # -inf fill, ties across chunks
    base[0, 3, :] = 3.0                                              # all equal
    tb = gu.make_builder(spec, w)
    got = gu.run(tb, spec, req, base=base)
    reps, trees = gu.compare(spec, w, req, got, base=base)
    for d, dep in enumerate(trees[0].depths_info):
        np.testing.assert_array_equal(got["cand_ids"][0, d], dep.cand, err_msg=f"depth {d}")
    _assert_ok(reps)
    tb.close()


def test_validate_rejects_nan(dev):
    import conditional_draft_tree_dominotree_amd as pkg
    spec = synth.small("nan", V=600, D=3, h=8, e=8, ds=8, r=8, M=4, k=2, N=6, group=501)
    spec, w, req = synth.workload(spec)
    base = req["base"].copy()
    base[0, 1, 17] = np.nan
    tb = gu.make_builder(spec, w)
    with pytest.raises(pkg.DtError) as ei:
        gu.run(tb, spec, req, base=base, flags=pkg.DT_VALIDATE)
    assert ei.value.status == pkg.binding.DT_EINVAL
    tb.close()


def test_runs_are_bitwise_reproducible(dev):
    spec = synth.small("repro", V=4000, D=6, h=64, e=64, ds=128, r=64, M=32, k=8, N=60, B=6,
                       wdtype="bf16", group=502, emb_std=0.5)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    a = gu.run(tb, spec, req)
    b = gu.run(tb, spec, req)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    tb.close()


@pytest.mark.parametrize("name", ["base", "batch3_fullv_T05"])
def test_marginal_flag_is_the_zero_correction_tree(dev, name):
    # DT_MARGINAL scores with the base logits alone: the oracle's tree with
    # W2 = 0 (itself pinned to an independent product-tree enumeration)
    import conditional_draft_tree_dominotree_amd as pkg
    kw = dict(SMALL)[name]
    spec = synth.small(name, group=300 + len(name), **kw)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    got = gu.run(tb, spec, req, flags=pkg.DT_MARGINAL)
    # a conditional build on the same handle afterwards (the marginal build
    # runs no workers; the exchange with them must still be in step)
    cond = gu.run(tb, spec, req)
    tb.close()
    w0 = dict(w)
    w0["w2"] = np.zeros_like(w["w2"])
    reps, trees = gu.compare(spec, w0, req, got)
    print(name, "marginal", gu.summarize(reps))
    _assert_ok(reps)
    assert all(r.exact for r in reps)
    reps, _ = gu.compare(spec, w, req, cond)
    _assert_ok(reps)


def test_marginal_with_root_state_bf16(dev):
    # a given root state changes nothing in the marginal scores
    import conditional_draft_tree_dominotree_amd as pkg
    spec = synth.small("marginal_root", V=3000, D=6, h=64, e=96, ds=1024, r=64, M=16, k=4, N=50, B=6,
                       wdtype="bf16", group=2201, emb_std=0.5, root_std=0.7)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    got = gu.run(tb, spec, req, flags=pkg.DT_ACT_BF16 | pkg.DT_MARGINAL)
    tb.close()
    w0 = dict(w)
    w0["w2"] = np.zeros_like(w["w2"])
    reps, _ = gu.compare(spec, w0, req, got)
    _assert_ok(reps)
    assert all(r.exact for r in reps)


@pytest.mark.parametrize("B,root", [(2, True), (3, False), (5, True)])
def test_bf16_register_workers_two_halves(dev, B, root):
    # the register workers serve the first ceil(B/2) requests of a step, then
    # the rest (16 nodes per request per step, so the first half fills whole
    # 16-column blocks); uneven halves, given and zero root states
    spec = synth.small(f"halves_b{B}", V=3000, D=7, h=64, e=96, ds=1024, r=64, M=16, k=4, N=80, B=B,
                       wdtype="bf16", group=1200 + B, emb_std=0.5, biases=True,
                       root_std=0.7 if root else 0.0)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    tb.set_schedule(halves=2, pops=16)
    got = gu.run(tb, spec, req)
    reps, trees = gu.compare(spec, w, req, got)
    print(gu.summarize(reps))
    _assert_ok(reps)
    gu.check_candidates(spec, trees, got, range(spec.B))
    tb.close()


def test_halves_alternate_on_one_handle(dev):
    # group flags carry 2 epoch + half in every launch, so a one-half build
    # after a two-half build (and back) waits for its own flags; each column's
    # product and state update do not depend on the split, so the trees are
    # bitwise the same
    spec = synth.small("halves_alt", V=3000, D=7, h=64, e=96, ds=1024, r=64, M=16, k=4, N=80, B=4,
                       wdtype="bf16", group=1290, emb_std=0.5, biases=True, root_std=0.7)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    outs = []
    for hv in (2, 1, 2, 1):
        tb.set_schedule(halves=hv, pops=16)
        outs.append(gu.run(tb, spec, req))
    reps, _ = gu.compare(spec, w, req, outs[0])
    print(gu.summarize(reps))
    _assert_ok(reps)
    for o in outs[1:]:
        for key in ("tokens", "parents", "depths", "scores", "n_nodes"):
            np.testing.assert_array_equal(o[key], outs[0][key], err_msg=key)
    tb.close()


def test_golden_tie_tree_through_the_gpu(dev):
    # the hand-worked tie fixture: equal logits, W2 = 0, every candidate
    # log-prob is -ln 2; pops tie on score and depth and are ordered by token,
    # then by the parent's index
    import json
    import math
    import os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_tree_ties.json")))
    V, D = fx["V"], fx["D"]
    spec = synth.small("golden_ties", V=V, D=D, h=8, e=8, ds=4, r=4, M=fx["M"], k=fx["k"], N=fx["N"],
                       T=fx["T"], group=1600, logits="zipf")    # the drawn logits are replaced below
    spec, w, req = synth.workload(spec)
    w = dict(w, w2=np.zeros_like(w["w2"]))
    base = np.array(fx["logits"], np.float32)[None]
    tb = gu.make_builder(spec, w)
    got = gu.run(tb, spec, req, base=base)
    tb.close()
    ex = fx["expected"]
    assert got["tokens"][0].tolist() == ex["tokens"]
    assert got["parents"][0].tolist() == ex["parents"]
    assert got["depths"][0].tolist() == ex["depths"]
    np.testing.assert_allclose(got["scores"][0], np.array(ex["scores_in_ln2"]) * math.log(2.0), rtol=0, atol=1e-6)


@pytest.mark.parametrize("wdtype,ds,B,M,k,N", [("f32", 64, 1, 8, 8, 120), ("f32", 64, 3, 8, 4, 90),
                                              ("bf16", 1024, 2, 8, 8, 150)])
def test_long_exact_tie_groups(dev, wdtype, ds, B, M, k, N):
    # W2 = 0 and every base logit equal: every child of a depth has the same
    # log-prob, so each depth's nodes form one exact tie group across all
    # parents (64 entries at depth 2 with k = 8, longer than a 32-entry pop
    # batch), ordered only by token and then by the parent's order
    spec = synth.small(f"longties_{wdtype}_{B}_{k}", V=96, D=4, h=64, e=96, ds=ds, r=64, M=M, k=k, N=N, B=B,
                       wdtype=wdtype, group=1700 + B + k, emb_std=0.5, biases=True, root_std=0.5)
    spec, w, req = synth.workload(spec)
    w = dict(w, w2=np.zeros_like(w["w2"]))
    base = np.zeros((B, spec.D, spec.V), np.float32)
    tb = gu.make_builder(spec, w)
    got = gu.run(tb, spec, req, base=base)
    tb.close()
    reps, trees = gu.compare(spec, w, req, got, base=base)
    print(gu.summarize(reps))
    gu.assert_parity(reps)
    assert all(r.exact for r in reps)
    for b, t in enumerate(trees):
        np.testing.assert_allclose(got["scores"][b, :N + 1], np.array(t.scores), rtol=0, atol=1e-5)
        # the largest group of equal (score, depth) really is longer than a
        # pop batch and spans several parents
        groups = {}
        for i in range(1, N + 1):
            groups.setdefault(t.depths[i], []).append(i)
        big = max(groups.values(), key=len)
        assert len(big) > 32 and len({t.parents[i] for i in big}) > 1
        assert len({t.scores[i] for i in big}) == 1


@pytest.mark.parametrize("V,M,k,N,zero_rows,dup", [
    (3000, 16, 4, 40, [(0, 1)], 0),          # one depth's hidden state zero: every logit 0
    (1000, 64, 8, 60, [(0, 0), (0, 2)], 0),  # vocabulary ending inside a 256-column tile, M = 64
    (5000, 8, 4, 30, [], 300),               # 300 equal W_lm columns: tie blocks across lists
    (2050, 1, 1, 10, [(1, 3)], 0),           # M = 1, two requests
])
def test_lm_head_fused_selection_edge_cases(dev, V, M, k, N, zero_rows, dup):
    # the LM head with the candidate selection in its epilogue: candidates,
    # their logits and the LSE against the oracle's own LM head and
    # selection, where equal logits force lists to be recomputed
    from oracle import ref
    B = 2 if any(b == 1 for b, _ in zero_rows) else 1
    spec = synth.small(f"lmsel_{V}_{M}_{dup}", V=V, D=4, h=128, e=64, ds=64, r=32, M=M, k=k, N=N, B=B,
                       wdtype="bf16", logits="lmhead", group=1800 + V + M, emb_std=0.5)
    spec, w, req = synth.workload(spec)
    w = dict(w)
    req = dict(req)
    hidden = req["hidden"].copy()
    for b, d in zero_rows:
        hidden[b, d] = 0
    req["hidden"] = hidden
    if dup:
        # column 7 scaled up (its logits lead the rows where they are
        # positive) and copied to 40 .. 40 + dup: ties that span lists
        wl = w["w_lm"].copy()
        wl[:, 7] = synth.bf16_bits(4.0 * synth.bits_to_f32(wl[:, 7]))
        wl[:, 40:40 + dup] = wl[:, 7:8]
        w["w_lm"] = wl
    tb = gu.make_builder(spec, w)
    import conditional_draft_tree_dominotree_amd as pkg
    o = tb.outputs(B, M, N, candidates=True, stats=True, logits=True)
    tb.build(gu.to_dev(hidden), None, None, top_m=M, top_k=k, budget=N, temperature=spec.T,
             flags=pkg.DT_ACT_BF16, out=o)
    tb.sync_status()
    got = {key: v.cpu().numpy() for key, v in o.items()}
    tb.close()
    rows = hidden.reshape(B * spec.D, spec.h)
    base = ref.lm_head_logits(rows, w["w_lm"], True).reshape(B, spec.D, V)
    assert np.max(np.abs(got["logits"].astype(np.float64) - base)) < 1e-4
    for b in range(B):
        for d in range(spec.D):
            dep = ref.candidates(base[b, d], M, spec.T)
            ids, vals = got["cand_ids"][b, d], got["cand_logits"][b, d]
            # the GPU's own logits at its candidates, in (value desc, id asc) order
            np.testing.assert_array_equal(vals, got["logits"][b, d, ids])
            assert all((vals[i] > vals[i + 1]) or (vals[i] == vals[i + 1] and ids[i] < ids[i + 1])
                       for i in range(M - 1)), (b, d)
            # and exactly the top M of those logits
            gl = got["logits"][b, d]
            order = np.lexsort((np.arange(V), -gl.astype(np.float64)))[:M]
            np.testing.assert_array_equal(ids, order, err_msg=f"request {b} depth {d}")
            if dep.margin >= 1e-4:
                np.testing.assert_array_equal(np.sort(ids), np.sort(dep.cand))
            assert abs(got["lse"][b, d] - dep.lse) <= 1e-4 * max(1.0, abs(dep.lse)), (b, d)
            if (b, d) in zero_rows:
                assert np.all(vals == 0) and np.array_equal(ids, np.arange(M))
    reps, trees = gu.compare(spec, w, req, got, base=base, logits_computed=True)
    print(gu.summarize(reps))
    gu.assert_parity(reps)
