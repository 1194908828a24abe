"""GPU parity of the greedy chain head (dt_draft_chain) with the oracle
(oracle/chain.py): the picked tokens bit-exact up to the first position
where the oracle's own pick had a runner-up within the float tolerance (a
near tie; the chains may then part), the corrected logits of the matched
picks within 1e-4 (fp32 weights) or 2e-2 (bf16 weights)."""
import numpy as np
import pytest

from oracle import chain, ref
from tests import gpu_util as gu
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    return torch.device("cuda:0")


def compare(spec, w, req, got, requests, base=None):
    bf16 = spec.wdtype == "bf16"
    tol = gu.TOL_BF16 if bf16 else gu.TOL_F32
    head = ref.make_head(w, bf16, spec.act_bf16)
    exact, ties = 0, 0
    for b in requests:
        hid = ref.hidden_values(req["hidden"][b], bf16)
        bl = base[b] if base is not None else req["base"][b]
        toks, logits, margins = chain.greedy_chain(head, bl, hid, req["root"][b])
        for d in range(spec.D):
            if got["tokens"][b, d] != toks[d]:
                assert margins[d] < tol, (b, d, got["tokens"][b, d], toks[d], margins[d])
                ties += 1
                break
            assert abs(float(got["logits"][b, d]) - logits[d]) <= tol, (b, d, got["logits"][b, d], logits[d])
        else:
            exact += 1
    return exact, ties


def run_chain(tb, spec, req, base=None):
    hidden = gu.to_dev(req["hidden"])
    if base is None and spec.logits != "lmhead":
        base = req["base"]
    root = gu.to_dev(req["root"]) if spec.root_std > 0 else None
    o = tb.chain(hidden, gu.to_dev(base), root)
    tb.sync_status()
    return {k: v.cpu().numpy() for k, v in o.items()}


def test_tiny(dev):
    spec, w, req = synth.workload("tiny")
    tb = gu.make_builder(spec, w)
    got = run_chain(tb, spec, req)
    tb.close()
    exact, ties = compare(spec, w, req, got, range(spec.B))
    assert exact == spec.B, (exact, ties)


def test_tiny_batch_root_state_and_ties(dev):
    # several requests with their own root states; one depth with an exact
    # tie in the base logits and W2 = 0 there is no correction to break it
    spec, w, req = synth.workload("tiny")
    rng = np.random.default_rng(5)
    B = 7
    req = {"base": np.repeat(req["base"], B, 0) + rng.normal(0, 1, (B, spec.D, spec.V)).astype(np.float32),
           "hidden": np.repeat(req["hidden"], B, 0), "root": rng.normal(0, 1, (B, spec.ds)).astype(np.float32)}
    w0 = dict(w)
    w0["w2"] = np.zeros_like(w["w2"])
    req["base"][3, 4, 10] = req["base"][3, 4, 900] = req["base"][3, 4].max() + 1.0
    spec = spec.replace(B=B, root_std=1.0)
    for weights in (w, w0):
        tb = gu.make_builder(spec, weights)
        got = run_chain(tb, spec, req)
        tb.close()
        exact, ties = compare(spec, weights, req, got, range(B))
        assert exact == B, (exact, ties)
    assert got["tokens"][3, 4] == 10


@pytest.mark.parametrize("name,sample", [("q4b_b1", [0]), ("q8b_b1", [0]), ("q8b_b32", [0, 13, 31])])
def test_full_shapes(dev, name, sample):
    spec, w, req = synth.workload(name)
    tb = gu.make_builder(spec, w)
    got = run_chain(tb, spec, req)
    tb.close()
    assert got["tokens"].shape == (spec.B, spec.D)
    assert np.all((got["tokens"] >= 0) & (got["tokens"] < spec.V))
    exact, ties = compare(spec, w, req, got, sample)
    print(name, f"{exact}/{len(sample)} chains exact, near-ties {ties}")
    assert exact + ties == len(sample)


def test_lm_head_route(dev):
    spec, w, req = synth.workload("q8b_lm")
    tb = gu.make_builder(spec, w)
    got = run_chain(tb, spec, req)
    tb.close()
    base = np.zeros((spec.B, spec.D, spec.V), np.float32)
    base[0] = ref.lm_head_logits(req["hidden"][0], w["w_lm"], True)
    exact, ties = compare(spec, w, req, got, [0], base=base)
    assert exact + ties == 1


@pytest.mark.parametrize("name,L", [("tiny", 1), ("tiny", 6), ("q8b_b1", 3)])
def test_fold_state(dev, name, L):
    import torch
    from oracle import chain as ochain
    spec, w, req = synth.workload(name)
    bf16 = spec.wdtype == "bf16"
    head = ref.make_head(w, bf16, spec.act_bf16)
    rng = np.random.default_rng(L)
    B = 5
    toks = rng.integers(0, spec.V, (B, L)).astype(np.int32)
    prev = rng.normal(0, 0.5, (B, spec.ds)).astype(np.float32)
    tb = gu.make_builder(spec, w, max_batch=B)
    got = tb.fold_state(torch.from_numpy(toks).cuda(), torch.from_numpy(prev).cuda())
    zero = tb.fold_state(torch.from_numpy(toks[:, :1].copy()).cuda())
    tb.sync_status()
    got, zero = got.cpu().numpy(), zero.cpu().numpy()
    tb.close()
    tol = 2e-3 if bf16 else 1e-5
    for b in range(B):
        want = ochain.fold_state(head, prev[b].astype(np.float64), toks[b])
        np.testing.assert_allclose(got[b], want, rtol=0, atol=tol, err_msg=f"request {b}")
        want0 = ochain.fold_state(head, np.zeros(spec.ds), toks[b, :1])
        np.testing.assert_allclose(zero[b], want0, rtol=0, atol=tol, err_msg=f"request {b} from zeros")


def test_fold_then_build(dev):
    # the folded state as the root state of a build: the tree equals the
    # oracle's tree from the oracle's folded state
    import torch
    from oracle import certify
    from oracle import chain as ochain
    spec, w, req = synth.workload("tiny")
    head = ref.make_head(w, False, False)
    toks = np.array([[5, 77, 1000]], np.int32)
    tb = gu.make_builder(spec, w)
    root = tb.fold_state(torch.from_numpy(toks).cuda())
    out = tb.build(gu.to_dev(req["hidden"]), gu.to_dev(req["base"]), root, top_m=spec.M, top_k=spec.k,
                   budget=spec.N, temperature=spec.T)
    tb.sync_status()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    tb.close()
    root_o = ochain.fold_state(head, np.zeros(spec.ds), toks[0])
    hid = req["hidden"][0].astype(np.float64)
    t = ref.build_tree(head, req["base"][0], hid, root_o, spec.M, spec.k, spec.N, spec.T, spec.norm)
    other = {k: got[k][0] for k in ("tokens", "parents", "depths", "scores")}
    other["n_nodes"] = int(got["n_nodes"][0])
    rep = certify.compare(t, head, hid, root_o, other, spec.k, spec.T, spec.norm, spec.N, gu.TOL_F32)
    assert rep.ok and rep.exact, rep


@pytest.mark.parametrize("B", [6, 9, 32])
def test_small_fp32_batches(dev, B):
    # every request-group width of the correction kernel (8, 16, 32), fp32
    # weights, a vocabulary that is not a multiple of the block size, random
    # root states
    spec = synth.small(f"chain_b{B}", group=700 + B, V=3001, D=5, h=32, e=24, ds=64, r=32, M=8, k=2, N=10,
                       B=B, root_std=0.5)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    got = run_chain(tb, spec, req)
    tb.close()
    exact, ties = compare(spec, w, req, got, range(B))
    assert exact == B, (exact, ties)


@pytest.mark.parametrize("B,V", [(5, 5003), (32, 4099)])
def test_small_bf16_odd_vocab(dev, B, V):
    # the matrix-core correction with a vocabulary that is neither a multiple
    # of 4 (unaligned base rows) nor of the 256-row block, up to 32 requests
    spec = synth.small(f"chain_bf16_{B}_{V}", group=800 + B, V=V, D=5, h=64, e=96, ds=128, r=64, M=8, k=2,
                       N=10, B=B, wdtype="bf16", emb_std=0.5, root_std=0.5)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    got = run_chain(tb, spec, req)
    tb.close()
    exact, ties = compare(spec, w, req, got, range(B))
    assert exact + ties == B, (exact, ties)
    assert exact >= B - 1, (exact, ties)


# ---- sampled chain (dt_draft_chain_sample) ---------------------------------

def compare_sampled(spec, w, req, got, requests, T, seed, base=None):
    """As compare(), against the oracle's Gumbel-max chain with the same seed:
    a pick may differ only where the oracle's perturbed scores had a
    runner-up within the float tolerance scaled by 1 / T."""
    bf16 = spec.wdtype == "bf16"
    tol = gu.TOL_BF16 if bf16 else gu.TOL_F32
    head = ref.make_head(w, bf16, spec.act_bf16)
    exact, ties = 0, 0
    for b in requests:
        hid = ref.hidden_values(req["hidden"][b], bf16)
        bl = base[b] if base is not None else req["base"][b]
        toks, logits, margins = chain.sampled_chain(head, bl, hid, req["root"][b], T, seed, b)
        for d in range(spec.D):
            if got["tokens"][b, d] != toks[d]:
                assert margins[d] < tol / T + 1e-5, (b, d, got["tokens"][b, d], toks[d], margins[d])
                ties += 1
                break
            assert abs(float(got["logits"][b, d]) - logits[d]) <= tol, (b, d, got["logits"][b, d], logits[d])
        else:
            exact += 1
    return exact, ties


def run_sampled(tb, spec, req, T, seed):
    hidden = gu.to_dev(req["hidden"])
    root = gu.to_dev(req["root"]) if spec.root_std > 0 else None
    o = tb.chain(hidden, gu.to_dev(req["base"]), root, temperature=T, seed=seed)
    tb.sync_status()
    return {k: v.cpu().numpy() for k, v in o.items()}


@pytest.mark.parametrize("T,seed", [(1.0, 7), (0.5, 2 ** 40 + 3)])
def test_sampled_tiny(dev, T, seed):
    spec, w, req = synth.workload("tiny")
    tb = gu.make_builder(spec, w)
    got = run_sampled(tb, spec, req, T, seed)
    again = run_sampled(tb, spec, req, T, seed)
    greedy = run_chain(tb, spec, req)
    tb.close()
    np.testing.assert_array_equal(got["tokens"], again["tokens"])
    exact, ties = compare_sampled(spec, w, req, got, range(spec.B), T, seed)
    assert exact == spec.B, (exact, ties)
    assert not np.array_equal(got["tokens"], greedy["tokens"])


@pytest.mark.parametrize("B,wdtype", [(9, "f32"), (32, "f32"), (5, "bf16"), (32, "bf16")])
def test_sampled_small_batches(dev, B, wdtype):
    # both correction kernels (fp32 rows; bf16 on the matrix cores), a
    # vocabulary that is not a multiple of 4, random root states; the row
    # index of each request keys its noise
    bf16 = wdtype == "bf16"
    kw = dict(h=64, e=96, ds=128, r=64, wdtype="bf16", emb_std=0.5) if bf16 else dict(h=32, e=24, ds=64, r=32)
    spec = synth.small(f"chain_smp_{B}_{wdtype}", group=900 + B + 50 * bf16, V=4001, D=5, M=8, k=2, N=10, B=B,
                       root_std=0.5, **kw)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    got = run_sampled(tb, spec, req, 0.8, 1234)
    other = run_sampled(tb, spec, req, 0.8, 1235)
    tb.close()
    exact, ties = compare_sampled(spec, w, req, got, range(B), 0.8, 1234)
    print(f"B={B} {wdtype}: {exact}/{B} sampled chains exact, near-ties {ties}")
    assert exact + ties == B and exact >= B - 1, (exact, ties)
    assert not np.array_equal(got["tokens"], other["tokens"])


def test_sampled_full_shape(dev):
    spec, w, req = synth.workload("q8b_b32")
    tb = gu.make_builder(spec, w)
    got = run_sampled(tb, spec, req, 1.0, 99)
    tb.close()
    assert np.all((got["tokens"] >= 0) & (got["tokens"] < spec.V))
    sample = [0, 13, 31]
    exact, ties = compare_sampled(spec, w, req, got, sample, 1.0, 99)
    print(f"q8b_b32 sampled: {exact}/{len(sample)} exact, near-ties {ties}")
    assert exact + ties == len(sample)


def test_sampled_refuses_bad_temperature(dev):
    import torch

    import conditional_draft_tree_dominotree_amd as pkg
    spec, w, req = synth.workload("tiny")
    tb = gu.make_builder(spec, w)
    hidden, base = gu.to_dev(req["hidden"]), gu.to_dev(req["base"])
    for T in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(pkg.DtError) as ei:
            tb.chain(hidden, base, temperature=T, seed=1)
        assert ei.value.status == pkg.binding.DT_EINVAL
    torch.cuda.synchronize()
    tb.close()
