"""dt_draft_chain_noalloc (the chain head with its workspace in the library's
fixed device array) against dt_draft_chain (the handle's workspace), both
called through the C ABI: two calls in a row, the second with a smaller
batch, must match the allocating entry point bit for bit."""
import ctypes

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


def _call(fn, tb, hidden, base, root, flags):
    import torch

    from conditional_draft_tree_dominotree_amd import binding
    b, D = hidden.shape[0], tb.dims.depths
    tokens = torch.full((b, D), -7, dtype=torch.int32, device=hidden.device)
    logits = torch.full((b, D), float("nan"), dtype=torch.float32, device=hidden.device)
    inp = binding.Inputs(b, base.data_ptr(), hidden.data_ptr(), None if root is None else root.data_ptr())
    fn(tb.handle, inp, flags, tokens.data_ptr(), logits.data_ptr(), tb.stream.cuda_stream)
    torch.cuda.synchronize()
    return tokens.cpu().numpy(), logits.cpu().numpy()


# bf16 with rank 64: the matrix-core correction; fp32: the FMA correction
@pytest.mark.parametrize("wdtype,ds", [("bf16", 1024), ("f32", 128)])
def test_noalloc_chain_matches_the_allocating_entry_point(dev, wdtype, ds):
    from conditional_draft_tree_dominotree_amd import binding
    spec = synth.small(f"noalloc_{wdtype}", V=5003, D=9, h=64, e=96, ds=ds, r=64, M=8, k=4, N=16, B=32,
                       wdtype=wdtype, group=1500 + ds, emb_std=0.5, biases=True, root_std=0.6)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    flags = binding.DT_ACT_BF16 if wdtype == "bf16" else 0
    hidden, base, root = gu.to_dev(req["hidden"]), gu.to_dev(req["base"]), gu.to_dev(req["root"])
    for b in (32, 7):      # the second call smaller: the array keeps the first call's values
        print(f"case: {wdtype} d_s={ds} batch {b}", flush=True)
        h, bl, r = hidden[:b].contiguous(), base[:b].contiguous(), root[:b].contiguous()
        want = _call(binding.dt_draft_chain, tb, h, bl, r, flags)
        got = _call(binding.dt_draft_chain_noalloc, tb, h, bl, r, flags)
        np.testing.assert_array_equal(got[0], want[0], err_msg=f"tokens, batch {b}")
        np.testing.assert_array_equal(got[1], want[1], err_msg=f"logits, batch {b}")
        assert np.all(want[0] >= 0) and np.all(np.isfinite(want[1]))
    tb.close()


def test_noalloc_chain_refusals(dev):
    import torch

    from conditional_draft_tree_dominotree_amd import binding
    # zero weights: the refusals come before any device work
    V, D, h, e, ds, r, B = 512, 2, 32, 32, 8192, 16, 32
    bf = dict(dtype=torch.bfloat16, device=dev)
    w = {"emb": torch.zeros(V, e, **bf), "w_ih": torch.zeros(3 * ds, e, **bf),
         "w_hh": torch.zeros(3 * ds, ds, **bf), "w1": torch.zeros(h + ds, r, **bf),
         "w2": torch.zeros(r, V, **bf)}
    import conditional_draft_tree_dominotree_amd as pkg
    tb = pkg.TreeBuilder(w, vocab=V, depths=D, hidden=h, emb_dim=e, state_dim=ds, rank=r, max_batch=B,
                         max_top_m=4, max_top_k=2, max_budget=4)
    hidden = torch.zeros(B, D, h, **bf)
    base = torch.zeros(B, D, V, dtype=torch.float32, device=dev)
    tokens = torch.zeros(B, D, dtype=torch.int32, device=dev)
    lib = binding.load_library()
    no_base = binding.Inputs(B, None, hidden.data_ptr(), None)
    assert lib.dt_draft_chain_noalloc(ctypes.c_void_p(tb.handle), ctypes.byref(no_base), binding.DT_ACT_BF16,
                                      ctypes.c_void_p(tokens.data_ptr()), None, None) == binding.DT_EINVAL
    # d_s = 8192 at batch 32 needs more than the 4 MiB array
    big = binding.Inputs(B, base.data_ptr(), hidden.data_ptr(), None)
    assert lib.dt_draft_chain_noalloc(ctypes.c_void_p(tb.handle), ctypes.byref(big), binding.DT_ACT_BF16,
                                      ctypes.c_void_p(tokens.data_ptr()), None, None) == binding.DT_EUNSUPPORTED
    assert "scratch" in pkg.dt_last_error()
    tb.close()
