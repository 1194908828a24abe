"""The C-ABI library loads and exports what include/dominotree.h declares;
argument errors are reported before any device work (no GPU needed)."""
import ctypes
import os
import re

import pytest

import conditional_draft_tree_dominotree_amd as pkg
from conditional_draft_tree_dominotree_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dominotree.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dt_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkg.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return pkg.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None


def test_version(lib):
    assert "gfx950" in pkg.dt_version()


def test_null_arguments_are_einval(lib):
    h = ctypes.c_void_p()
    assert lib.dt_create(None, None, None, None, None) == binding.DT_EINVAL
    assert lib.dt_create(ctypes.byref(h), None, None, None, None) == binding.DT_EINVAL
    assert "required" in pkg.dt_last_error()
    assert lib.dt_build_trees(None, None, None, None, None) == binding.DT_EINVAL
    assert lib.dt_sync_status(None, None) == binding.DT_EINVAL
    assert lib.dt_destroy(None) == binding.DT_OK


@pytest.mark.parametrize("dims,params,code", [
    ((0, 7, 8, 8, 8, 4, 1), (4, 2, 8, 1.0), binding.DT_EINVAL),          # vocab 0
    ((64, 7, 8, 8, 8, 4, 33), (4, 2, 8, 1.0), binding.DT_EUNSUPPORTED),  # batch > 32
    ((1048575, 7, 8, 8, 8, 4, 1), (4, 2, 8, 1.0), binding.DT_EUNSUPPORTED),  # vocab > 2^20 - 2
    ((64, 40, 8, 8, 8, 4, 1), (4, 2, 8, 1.0), binding.DT_EUNSUPPORTED),  # depths > 31
    ((64, 7, 8, 8, 8, 4, 1), (0, 1, 8, 1.0), binding.DT_EINVAL),         # M = 0
    ((64, 7, 8, 8, 8, 4, 1), (65, 2, 8, 1.0), binding.DT_EINVAL),        # M > V
    ((128, 7, 8, 8, 8, 4, 1), (65, 2, 8, 1.0), binding.DT_EUNSUPPORTED), # M > 64
    ((64, 7, 8, 8, 8, 4, 1), (4, 5, 8, 1.0), binding.DT_EINVAL),         # k > M
    ((64, 7, 8, 8, 8, 4, 1), (4, 2, 0, 1.0), binding.DT_EINVAL),         # N = 0
    ((64, 7, 8, 8, 8, 4, 1), (4, 2, 2000, 1.0), binding.DT_EUNSUPPORTED),  # N > 1024
    ((64, 7, 8, 8, 8, 4, 1), (64, 64, 1000, 1.0), binding.DT_EUNSUPPORTED),  # frontier
    ((64, 7, 8, 8, 8, 4, 1), (4, 2, 8, 0.0), binding.DT_EINVAL),         # T = 0
    ((64, 7, 8, 8, 8, 4, 1), (4, 2, 8, float("nan")), binding.DT_EINVAL),
])
def test_argument_errors_before_device_work(lib, dims, params, code):
    d = binding.Dims(*dims, binding.DT_F32)
    # non-null fake pointers: validation must fail before they are touched
    w = binding.Weights(16, 16, 16, None, None, 16, 16, None)
    p = binding.Params(*params, binding.DT_NORM_TOPM, 0)
    h = ctypes.c_void_p()
    assert lib.dt_create(ctypes.byref(h), ctypes.byref(d), ctypes.byref(w), ctypes.byref(p),
                         None) == code
    assert h.value is None
    assert pkg.dt_last_error()


def test_missing_weight_is_einval(lib):
    d = binding.Dims(64, 7, 8, 8, 8, 4, 1, binding.DT_F32)
    w = binding.Weights(16, None, 16, None, None, 16, 16, None)
    p = binding.Params(4, 2, 8, 1.0, binding.DT_NORM_TOPM, 0)
    h = ctypes.c_void_p()
    assert lib.dt_create(ctypes.byref(h), ctypes.byref(d), ctypes.byref(w), ctypes.byref(p),
                         None) == binding.DT_EINVAL


def test_unknown_flags_are_einval(lib):
    d = binding.Dims(64, 7, 8, 8, 8, 4, 1, binding.DT_F32)
    w = binding.Weights(16, 16, 16, None, None, 16, 16, None)
    p = binding.Params(4, 2, 8, 1.0, binding.DT_NORM_TOPM, 0x80)
    h = ctypes.c_void_p()
    assert lib.dt_create(ctypes.byref(h), ctypes.byref(d), ctypes.byref(w), ctypes.byref(p),
                         None) == binding.DT_EINVAL


@pytest.mark.parametrize("view,out,code", [
    ((0, 9, 16, 16, 16, 16), (16, 16, None), binding.DT_EINVAL),           # batch 0
    ((2, 0, 16, 16, 16, 16), (16, 16, None), binding.DT_EINVAL),           # cols 0
    ((2, 1026, 16, 16, 16, 16), (16, 16, None), binding.DT_EUNSUPPORTED),  # cols > N_max + 1
    ((2, 9, None, 16, 16, 16), (16, 16, None), binding.DT_EINVAL),         # no parents
    ((2, 9, 16, None, 16, 16), (16, 16, None), binding.DT_EINVAL),         # no depths
    ((2, 9, 16, 16, 16, None), (16, 16, None), binding.DT_EINVAL),         # no n_nodes
    ((2, 9, 16, 16, 16, 16), (None, 16, None), binding.DT_EINVAL),         # no mask
    ((2, 9, 16, 16, 16, 16), (16, None, None), binding.DT_EINVAL),         # no positions
    ((2, 9, 16, 16, None, 16), (16, 16, 16), binding.DT_EINVAL),           # flat tokens need tokens
])
def test_tree_attention_argument_errors(lib, view, out, code):
    b, cols, par, dep, tok, nn = view
    v = binding.TreeView(b, cols, par, dep, tok, nn, None, None)
    o = binding.VerifyOutputs(out[0], out[1], out[2], None)
    assert lib.dt_tree_attention_inputs(ctypes.byref(v), ctypes.byref(o), None) == code
    assert pkg.dt_last_error()
    assert lib.dt_tree_attention_inputs(None, None, None) == binding.DT_EINVAL


def test_chain_null_arguments_are_einval(lib):
    assert lib.dt_draft_chain(None, None, 0, None, None, None) == binding.DT_EINVAL
    assert "required" in pkg.dt_last_error()
    assert lib.dt_draft_chain_sample(None, None, 0, 1.0, 1, None, None, None) == binding.DT_EINVAL
    assert "required" in pkg.dt_last_error()


def test_fold_null_arguments_are_einval(lib):
    assert lib.dt_fold_state(None, 1, 1, None, None, None, 0, None) == binding.DT_EINVAL
    assert "required" in pkg.dt_last_error()


def test_schedule_and_error_hook_null_arguments(lib):
    s = binding.Schedule(0, 0, 0, 0)
    assert lib.dt_set_schedule(None, ctypes.byref(s)) == binding.DT_EINVAL
    assert lib.dt_set_device_error(None, 1, None) == binding.DT_EINVAL
    assert "NULL" in pkg.dt_last_error()


# ----------------------------------------------------------------------------
# the torch layer refuses tensors the library would misread, before any
# pointer reaches the C ABI (checked here with host tensors: dtype and shape
# are checked before the device)

torch = pytest.importorskip("torch")

V, D, H, E, DS, R, BMAX = 64, 3, 16, 8, 4, 8, 4


def _weights(dtype=torch.float32, **over):
    w = {"emb": torch.zeros(V, E), "w_ih": torch.zeros(3 * DS, E), "w_hh": torch.zeros(3 * DS, DS),
         "w1": torch.zeros(H + DS, R), "w2": torch.zeros(R, V)}
    w = {k: v.to(dtype) for k, v in w.items()}
    w.update(over)
    return w


def _builder_kwargs():
    return dict(vocab=V, depths=D, hidden=H, emb_dim=E, state_dim=DS, rank=R, max_batch=BMAX,
                max_top_m=4, max_top_k=2, max_budget=8)


@pytest.mark.parametrize("over,msg", [
    ({"w2": torch.zeros(R, V + 1)}, "shape"),
    ({"w_hh": torch.zeros(3 * DS, DS, dtype=torch.bfloat16)}, "float32"),
    ({"b_ih": torch.zeros(3 * DS, dtype=torch.bfloat16)}, "float32"),
    ({"b_hh": torch.zeros(3 * DS + 1)}, "shape"),
    ({"w_lm": torch.zeros(H, V - 1)}, "shape"),
    ({"w1": torch.zeros(R, H + DS).t()}, "contiguous"),
    ({}, "device"),
])
def test_builder_refuses_bad_weights(over, msg):
    with pytest.raises(ValueError, match=msg):
        binding.TreeBuilder(_weights(**over), **_builder_kwargs())


def _unbound_builder():
    # the argument checks of a builder, without a handle
    tb = object.__new__(binding.TreeBuilder)
    tb.torch = torch
    tb.dims = binding.Dims(V, D, H, E, DS, R, BMAX, binding.DT_F32)
    tb.tdtype = torch.float32
    tb.wdtype = binding.DT_F32
    tb.device = torch.device("cpu")
    return tb


@pytest.mark.parametrize("hidden,base,root,msg", [
    (torch.zeros(2, D, H), torch.zeros(2, D, V, dtype=torch.bfloat16), None, "float32"),
    (torch.zeros(2, D, H), torch.zeros(2, D, V - 1), None, "shape"),
    (torch.zeros(2, D + 1, H), None, None, "shape"),
    (torch.zeros(2, D, H, dtype=torch.bfloat16), None, None, "float32"),
    (torch.zeros(2, D, H), None, torch.zeros(3, DS), "shape"),
    (torch.zeros(BMAX + 1, D, H), None, None, "batch"),
    (torch.zeros(2, H), None, None, "hidden"),
    (torch.zeros(2, D, H), torch.zeros(2, D, V), None, "device"),
])
def test_build_refuses_bad_inputs(hidden, base, root, msg):
    tb = _unbound_builder()
    with pytest.raises(ValueError, match=msg):
        tb.build(hidden, base, root, top_m=4, top_k=2, budget=8)
    with pytest.raises(ValueError, match=msg):
        tb.chain(hidden, base, root)


def test_output_refusal():
    # budget 8 needs 9 columns per request
    with pytest.raises(ValueError, match="output tokens"):
        binding._check_tensor("output tokens", torch.zeros(2, 8, dtype=torch.int32), torch.int32, (2, 9))


def test_fold_refuses_bad_tokens():
    tb = _unbound_builder()
    with pytest.raises(ValueError, match="int32"):
        tb.fold_state(torch.zeros(2, 5, dtype=torch.int64))
    with pytest.raises(ValueError, match="shape"):
        tb.fold_state(torch.zeros(2, 5, dtype=torch.int32), torch.zeros(2, DS + 1))


def test_tree_attention_refuses_bad_shapes():
    p = torch.zeros(2, 9, dtype=torch.int32)
    with pytest.raises(ValueError, match="shape"):
        pkg.tree_attention_inputs(p, torch.zeros(2, 8, dtype=torch.int32), torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="int32"):
        pkg.tree_attention_inputs(p, p, torch.zeros(2, dtype=torch.int64))
