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


def test_fold_null_arguments_are_einval(lib):
    assert lib.dt_fold_state(None, 1, 1, None, None, None, 0, None) == binding.DT_EINVAL
    assert "required" in pkg.dt_last_error()
