"""GPU tests of the boundary's contract with its caller: the work is enqueued
on the caller's stream, a build allocates no device memory, and a schedule
that needs more blocks than the device holds at once is refused."""
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


def _builder(spec, w, stream=None):
    import conditional_draft_tree_dominotree_amd as pkg
    tw = {k: gu.to_dev(v) for k, v in w.items()}
    return pkg.TreeBuilder(tw, vocab=spec.V, depths=spec.D, hidden=spec.h, emb_dim=spec.e, state_dim=spec.ds,
                           rank=spec.r, max_batch=spec.B, max_top_m=spec.M, max_top_k=spec.k, max_budget=spec.N,
                           stream=stream)


KEYS = ("tokens", "parents", "depths", "scores", "n_nodes")


def test_build_runs_in_order_on_the_callers_stream(dev):
    # the inputs are written on the builder's stream behind a long spin; a
    # build enqueued after them on that stream must read them, not the zeros
    # the buffers held when the host issued the build
    import torch

    import conditional_draft_tree_dominotree_amd as pkg
    spec = synth.small("stream_order", V=3000, D=6, h=64, e=96, ds=1024, r=64, M=16, k=4, N=40, B=4,
                       wdtype="bf16", group=2101, emb_std=0.5)
    spec, w, req = synth.workload(spec)
    s = torch.cuda.Stream()
    tb = _builder(spec, w, stream=s)
    with torch.cuda.stream(s):
        want = gu.run(tb, spec, req)
    reps, _ = gu.compare(spec, w, req, want)
    gu.assert_parity(reps)

    src_h, src_b = gu.to_dev(req["hidden"]), gu.to_dev(req["base"])
    hidden, base = torch.zeros_like(src_h), torch.zeros_like(src_b)
    out = tb.outputs(spec.B, spec.M, spec.N)
    for v in out.values():
        v.fill_(7)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        torch.cuda._sleep(20_000_000)  # some milliseconds of spinning on s
        hidden.copy_(src_h)
        base.copy_(src_b)
    kw = dict(top_m=spec.M, top_k=spec.k, budget=spec.N, temperature=spec.T, flags=pkg.DT_ACT_BF16)
    tb.build(hidden, base, **kw, out=out)
    # the outputs are not complete before the stream reaches the build
    done = torch.cuda.Event()
    done.record(s)
    torch.cuda.current_stream().wait_event(done)
    got = {k: v.cpu().numpy() for k, v in out.items()}
    tb.sync_status()
    for key in KEYS:
        np.testing.assert_array_equal(got[key], want[key], err_msg=key)
    tb.close()


def test_build_allocates_no_device_memory(dev):
    import torch

    import conditional_draft_tree_dominotree_amd as pkg
    spec, w, req = synth.workload("tiny")
    tb = gu.make_builder(spec, w)
    hidden, base = gu.to_dev(req["hidden"]), gu.to_dev(req["base"])
    flags = pkg.DT_ACT_BF16 if spec.wdtype == "bf16" else 0
    kw = dict(top_m=spec.M, top_k=spec.k, budget=spec.N, temperature=spec.T, flags=flags)
    out = tb.outputs(spec.B, spec.M, spec.N, candidates=True, stats=True)
    for _ in range(3):
        tb.build(hidden, base, **kw, out=out)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(50):
        tb.build(hidden, base, **kw, out=out)
    torch.cuda.synchronize()
    tb.sync_status()
    assert torch.cuda.mem_get_info()[0] == free0
    tb.close()


def test_more_blocks_than_compute_units_is_refused(dev):
    # one weight tile per worker at d_s = 1024, r = 544: (3 * 1024 + 544) / 16
    # = 226 workers beside 32 requests, more blocks than the device's compute
    # units, which a build needs resident at once; the default schedule packs
    # two tiles into a worker and builds
    import torch

    import conditional_draft_tree_dominotree_amd as pkg
    spec = synth.small("occupancy", V=2000, D=5, h=64, e=96, ds=1024, r=544, M=8, k=3, N=24, B=32,
                       wdtype="bf16", group=2102, emb_std=0.5)
    spec, w, req = synth.workload(spec)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert (3 * spec.ds + spec.r) // 16 + spec.B > n_cu
    tb = gu.make_builder(spec, w)
    tb.set_schedule(lds_workers=1, tiles_per_worker=1)
    hidden, base = gu.to_dev(req["hidden"]), gu.to_dev(req["base"])
    with pytest.raises(pkg.DtError) as ei:
        tb.build(hidden, base, top_m=spec.M, top_k=spec.k, budget=spec.N, temperature=spec.T,
                 flags=pkg.DT_ACT_BF16)
    assert ei.value.status == pkg.binding.DT_EUNSUPPORTED
    tb.set_schedule()
    got = gu.run(tb, spec, req)
    reps, _ = gu.compare(spec, w, req, got)
    gu.assert_parity(reps)
    tb.close()
