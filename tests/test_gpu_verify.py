"""GPU parity of the tree-attention inputs (dt_tree_attention_inputs) with
the oracle (oracle/verify.py), bit-exact: random valid trees at the builder's
output shapes (budget 32, 128, 256 and the largest, 1024), ragged and empty
trees, broken trees, and trees built by the library itself."""
import numpy as np
import pytest

from oracle import verify
from tests import gpu_util as gu
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    return torch.device("cuda:0")


def random_trees(seed, b, cols, ns):
    rng = np.random.default_rng(seed)
    par = np.full((b, cols), -1, np.int32)
    dep = np.full((b, cols), -1, np.int32)
    tok = np.full((b, cols), -1, np.int32)
    for r in range(b):
        dep[r, 0] = 0
        for i in range(1, ns[r] + 1):
            # mostly shallow, sometimes a long chain (depth up to ~31 when cols allow)
            par[r, i] = i - 1 if rng.random() < 0.2 else rng.integers(max(0, i - 40), i)
            dep[r, i] = dep[r, par[r, i]] + 1
            tok[r, i] = rng.integers(0, 151936)
    return par, dep, tok


def run_gpu(par, dep, tok, nn, prefix=None, anchor=None, with_tokens=True):
    import torch
    import conditional_draft_tree_dominotree_amd as pkg
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    o = pkg.tree_attention_inputs(t(par), t(dep), t(nn), tokens=t(tok) if with_tokens else None,
                                  prefix_len=t(prefix), anchor=t(anchor))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def check(par, dep, tok, nn, prefix, anchor, got, with_tokens=True):
    b, cols = par.shape
    for r in range(b):
        mask, pos, flat, bad = verify.tree_attention_inputs(
            par[r], dep[r], tok[r], int(nn[r]), 0 if prefix is None else int(prefix[r]),
            -1 if anchor is None else int(anchor[r]))
        np.testing.assert_array_equal(got["mask"][r].view(np.uint32), verify.pack_mask(mask),
                                      err_msg=f"tree {r}")
        np.testing.assert_array_equal(got["positions"][r], pos, err_msg=f"tree {r}")
        if with_tokens:
            np.testing.assert_array_equal(got["tokens"][r], flat, err_msg=f"tree {r}")
        assert int(got["bad"][r]) == int(bad), (r, got["bad"][r], bad)


@pytest.mark.parametrize("b,cols", [(1, 9), (32, 33), (32, 129), (32, 257), (4, 1025), (3, 1)])
def test_random_trees(dev, b, cols):
    rng = np.random.default_rng(cols)
    ns = [cols - 1] * b
    if b > 2:
        ns[1] = 0                              # an empty tree (root only)
        ns[2] = int(rng.integers(0, cols))     # a ragged one
    par, dep, tok = random_trees(cols + b, b, cols, ns)
    nn = np.array(ns, np.int32)
    prefix = rng.integers(0, 4096, b).astype(np.int32)
    anchor = rng.integers(0, 151936, b).astype(np.int32)
    got = run_gpu(par, dep, tok, nn, prefix, anchor)
    check(par, dep, tok, nn, prefix, anchor, got)
    print(f"b={b} cols={cols}: bit-exact, max depth {int(dep.max())}")


def test_optional_inputs_absent(dev):
    par, dep, tok = random_trees(5, 6, 65, [64, 10, 0, 64, 33, 1])
    nn = np.array([64, 10, 0, 64, 33, 1], np.int32)
    got = run_gpu(par, dep, tok, nn, None, None, with_tokens=False)
    assert "tokens" not in got
    check(par, dep, tok, nn, None, None, got, with_tokens=False)


def test_broken_trees_are_flagged(dev):
    b, cols = 6, 17
    par, dep, tok = random_trees(9, b, cols, [12] * b)
    nn = np.array([12] * b, np.int32)
    par[0, 7] = 9          # a parent not smaller than its child
    dep[1, 5] += 1         # a depth other than the path length
    nn[2] = 17             # n_nodes past the last column
    nn[3] = -3             # negative n_nodes
    par[4, 0] = 0          # a root with a parent
    got = run_gpu(par, dep, tok, nn)
    check(par, dep, tok, nn, None, None, got)
    np.testing.assert_array_equal(got["bad"], [1, 1, 1, 1, 1, 0])


def test_on_built_trees(dev):
    # the library's own trees (tiny workload) go straight from the builder's
    # outputs into the verification inputs
    import torch
    import conditional_draft_tree_dominotree_amd as pkg
    spec, w, req = synth.workload("tiny")
    tb = gu.make_builder(spec, w)
    out = tb.build(gu.to_dev(req["hidden"]), gu.to_dev(req["base"]), top_m=spec.M, top_k=spec.k,
                   budget=spec.N, temperature=spec.T)
    prefix = torch.tensor([37], dtype=torch.int32, device="cuda")
    anchor = torch.tensor([3], dtype=torch.int32, device="cuda")
    o = pkg.tree_attention_inputs(out["parents"], out["depths"], out["n_nodes"], tokens=out["tokens"],
                                  prefix_len=prefix, anchor=anchor, stream=tb.stream)
    tb.sync_status()
    got = {k: v.cpu().numpy() for k, v in o.items()}
    host = {k: v.cpu().numpy() for k, v in out.items()}
    tb.close()
    check(host["parents"], host["depths"], host["tokens"], host["n_nodes"], np.array([37]), np.array([3]),
          got)
    assert got["bad"][0] == 0
