"""GPU tests of the boundary's failure path.

The failure is forced from the host: dt_set_device_error writes the handle's
device error word before a build, as a builder wait that ran out would.  No
kernel faults or hangs: every wait of the build is bounded and gives up at its
next periodic look at the word, so the launch ends normally.
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


@pytest.mark.parametrize("wdtype,ds", [("f32", 64), ("bf16", 1024)])
def test_device_error_is_reported_then_reset(dev, wdtype, ds):
    import torch

    import conditional_draft_tree_dominotree_amd as pkg
    spec = synth.small(f"err_{wdtype}", V=3000, D=6, h=64, e=96, ds=ds, r=64, M=16, k=4, N=60, B=4,
                       wdtype=wdtype, group=1400 + ds, emb_std=0.5)
    spec, w, req = synth.workload(spec)
    tb = gu.make_builder(spec, w)
    first = gu.run(tb, spec, req)
    reps, _ = gu.compare(spec, w, req, first)
    gu.assert_parity(reps)

    # a build launched with the error word set: it ends, and its controllers
    # copy the word to the host mirror
    print(f"case: {wdtype} d_s={ds}, error word preset", flush=True)
    tb.set_device_error(3)
    hidden, base = gu.to_dev(req["hidden"]), gu.to_dev(req["base"])
    flags = pkg.DT_ACT_BF16 if wdtype == "bf16" else 0
    kw = dict(top_m=spec.M, top_k=spec.k, budget=spec.N, temperature=spec.T, flags=flags)
    tb.build(hidden, base, **kw)
    torch.cuda.synchronize()
    # the next build call refuses without enqueuing anything
    with pytest.raises(pkg.DtError) as ei:
        tb.build(hidden, base, **kw)
    assert ei.value.status == pkg.binding.DT_EDEVICE
    # dt_sync_status reports the failure once and resets the handle
    with pytest.raises(pkg.DtError) as ei:
        tb.sync_status()
    assert ei.value.status == pkg.binding.DT_EDEVICE and "reset" in str(ei.value)
    tb.sync_status()
    # builds after the reset return the first build's trees bit for bit
    for _ in range(2):
        again = gu.run(tb, spec, req)
        for key in ("tokens", "parents", "depths", "scores", "n_nodes"):
            np.testing.assert_array_equal(again[key], first[key], err_msg=key)
    tb.close()


def test_schedule_rejects_out_of_range(dev):
    import conditional_draft_tree_dominotree_amd as pkg
    spec, w, req = synth.workload("tiny")
    tb = gu.make_builder(spec, w)
    for kw in (dict(pops=17), dict(halves=3), dict(lds_workers=2), dict(tiles_per_worker=-1),
               dict(dl=2), dict(exchange=2), dict(launch=3)):
        with pytest.raises(pkg.DtError) as ei:
            tb.set_schedule(**kw)
        assert ei.value.status == pkg.binding.DT_EINVAL
    tb.set_schedule(pops=4)
    got = gu.run(tb, spec, req)
    reps, _ = gu.compare(spec, w, req, got)
    gu.assert_parity(reps)
    tb.close()
