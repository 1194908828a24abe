"""ctypes binding of libdominotree.so (argument marshalling only).

The functions dt_create / dt_build_trees / dt_sync_status / dt_phase_times /
dt_destroy / dt_tree_attention_inputs / dt_last_error / dt_version mirror
include/dominotree.h one to one; TreeBuilder and tree_attention_inputs wrap
them for torch device tensors.  Every step of the
build runs in the HIP library: when it is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))

DT_OK, DT_EINVAL, DT_EUNSUPPORTED, DT_ENOMEM, DT_EHIP, DT_EDEVICE = 0, -1, -2, -3, -4, -5
DT_F32, DT_BF16 = 0, 1
DT_NORM_TOPM, DT_NORM_FULLV = 0, 1
DT_ACT_BF16, DT_VALIDATE, DT_TIMING, DT_MARGINAL = 1, 2, 4, 8
_STATUS = {0: "DT_OK", -1: "DT_EINVAL", -2: "DT_EUNSUPPORTED", -3: "DT_ENOMEM", -4: "DT_EHIP",
           -5: "DT_EDEVICE"}


class DtError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class Dims(C.Structure):
    _fields_ = [("vocab", C.c_int32), ("depths", C.c_int32), ("hidden", C.c_int32),
                ("emb_dim", C.c_int32), ("state_dim", C.c_int32), ("rank", C.c_int32),
                ("max_batch", C.c_int32), ("wdtype", C.c_int)]


class Weights(C.Structure):
    _fields_ = [("emb", C.c_void_p), ("w_ih", C.c_void_p), ("w_hh", C.c_void_p),
                ("b_ih", C.c_void_p), ("b_hh", C.c_void_p), ("w1", C.c_void_p),
                ("w2", C.c_void_p), ("w_lm", C.c_void_p)]


class Params(C.Structure):
    _fields_ = [("top_m", C.c_int32), ("top_k", C.c_int32), ("budget", C.c_int32),
                ("temperature", C.c_float), ("norm", C.c_int), ("flags", C.c_uint32)]


class Inputs(C.Structure):
    _fields_ = [("batch", C.c_int32), ("base_logits", C.c_void_p), ("hidden", C.c_void_p),
                ("root_state", C.c_void_p)]


class Outputs(C.Structure):
    _fields_ = [("tokens", C.c_void_p), ("parents", C.c_void_p), ("depths", C.c_void_p),
                ("scores", C.c_void_p), ("n_nodes", C.c_void_p), ("cand_ids", C.c_void_p),
                ("cand_logits", C.c_void_p), ("lse", C.c_void_p)]


class TreeView(C.Structure):
    _fields_ = [("batch", C.c_int32), ("cols", C.c_int32), ("parents", C.c_void_p),
                ("depths", C.c_void_p), ("tokens", C.c_void_p), ("n_nodes", C.c_void_p),
                ("prefix_len", C.c_void_p), ("anchor", C.c_void_p)]


class VerifyOutputs(C.Structure):
    _fields_ = [("mask", C.c_void_p), ("positions", C.c_void_p), ("tokens", C.c_void_p),
                ("bad", C.c_void_p)]


EXPORTS = ["dt_create", "dt_build_trees", "dt_sync_status", "dt_phase_times", "dt_destroy",
           "dt_last_error", "dt_version", "dt_tree_attention_inputs", "dt_draft_chain", "dt_fold_state"]
_lib = None


def library_path() -> str:
    return os.path.join(PKG, "libdominotree.so")


def load_library():
    """Load libdominotree.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build()")
    lib = C.CDLL(path)
    lib.dt_create.restype = C.c_int
    lib.dt_create.argtypes = [C.POINTER(C.c_void_p), C.POINTER(Dims), C.POINTER(Weights),
                              C.POINTER(Params), C.c_void_p]
    lib.dt_build_trees.restype = C.c_int
    lib.dt_build_trees.argtypes = [C.c_void_p, C.POINTER(Inputs), C.POINTER(Params),
                                   C.POINTER(Outputs), C.c_void_p]
    lib.dt_sync_status.restype = C.c_int
    lib.dt_sync_status.argtypes = [C.c_void_p, C.c_void_p]
    lib.dt_phase_times.restype = C.c_int
    lib.dt_phase_times.argtypes = [C.c_void_p, C.POINTER(C.c_float), C.c_int,
                                   C.POINTER(C.c_int32)]
    lib.dt_destroy.restype = C.c_int
    lib.dt_destroy.argtypes = [C.c_void_p]
    lib.dt_last_error.restype = C.c_char_p
    lib.dt_last_error.argtypes = []
    lib.dt_version.restype = C.c_char_p
    lib.dt_version.argtypes = []
    lib.dt_draft_chain.restype = C.c_int
    lib.dt_draft_chain.argtypes = [C.c_void_p, C.POINTER(Inputs), C.c_uint32, C.c_void_p, C.c_void_p,
                                   C.c_void_p]
    lib.dt_fold_state.restype = C.c_int
    lib.dt_fold_state.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_uint32, C.c_void_p]
    lib.dt_tree_attention_inputs.restype = C.c_int
    lib.dt_tree_attention_inputs.argtypes = [C.POINTER(TreeView), C.POINTER(VerifyOutputs), C.c_void_p]
    _lib = lib
    return lib


def _check(status: int):
    if status != DT_OK:
        raise DtError(status, dt_last_error())


def dt_last_error() -> str:
    return load_library().dt_last_error().decode()


def dt_version() -> str:
    return load_library().dt_version().decode()


def dt_create(dims: Dims, weights: Weights, max_params: Params, stream: int = 0) -> int:
    h = C.c_void_p()
    _check(load_library().dt_create(C.byref(h), C.byref(dims), C.byref(weights),
                                    C.byref(max_params), C.c_void_p(stream)))
    return h.value


def dt_build_trees(handle: int, inputs: Inputs, params: Params, outputs: Outputs, stream: int = 0):
    _check(load_library().dt_build_trees(C.c_void_p(handle), C.byref(inputs), C.byref(params),
                                         C.byref(outputs), C.c_void_p(stream)))


def dt_sync_status(handle: int, stream: int = 0):
    _check(load_library().dt_sync_status(C.c_void_p(handle), C.c_void_p(stream)))


PHASES = ["lm_head_or_P", "candidates", "P_join", "builder_setup", "tree_kernel"]


def dt_phase_times(handle: int) -> tuple:
    """(mean ms per phase, in PHASES order, builds averaged)."""
    ms = (C.c_float * len(PHASES))()
    cnt = C.c_int32()
    _check(load_library().dt_phase_times(C.c_void_p(handle), ms, len(PHASES), C.byref(cnt)))
    return list(ms), cnt.value


def dt_destroy(handle: int):
    _check(load_library().dt_destroy(C.c_void_p(handle)))


def dt_draft_chain(handle: int, inputs: Inputs, flags: int, tokens: int, logits, stream: int = 0):
    _check(load_library().dt_draft_chain(C.c_void_p(handle), C.byref(inputs), C.c_uint32(flags),
                                         C.c_void_p(tokens), C.c_void_p(logits), C.c_void_p(stream)))


def dt_fold_state(handle: int, batch: int, n_tokens: int, tokens: int, prev_state, state_out: int,
                  flags: int, stream: int = 0):
    _check(load_library().dt_fold_state(C.c_void_p(handle), batch, n_tokens, C.c_void_p(tokens),
                                        C.c_void_p(prev_state), C.c_void_p(state_out), C.c_uint32(flags),
                                        C.c_void_p(stream)))


def dt_tree_attention_inputs(view: TreeView, out: VerifyOutputs, stream: int = 0):
    _check(load_library().dt_tree_attention_inputs(C.byref(view), C.byref(out), C.c_void_p(stream)))


# ----------------------------------------------------------------------------
# torch convenience layer


def _ptr(t):
    return None if t is None else t.data_ptr()


class TreeBuilder:
    """A handle plus caller-owned output tensors, for torch device tensors.

    weights: dict with emb, w_ih, w_hh, w1, w2 (torch.float32 or torch.bfloat16,
    contiguous, on the device) and optional b_ih, b_hh (float32) and w_lm.
    """

    def __init__(self, weights: dict, *, vocab, depths, hidden, emb_dim, state_dim, rank,
                 max_batch, max_top_m, max_top_k, max_budget, stream=None):
        import torch
        self.torch = torch
        w = {k: v for k, v in weights.items() if v is not None}
        dt = w["w_ih"].dtype
        self.wdtype = DT_BF16 if dt == torch.bfloat16 else DT_F32
        for k, v in w.items():
            if not v.is_cuda or not v.is_contiguous():
                raise ValueError(f"weight {k} must be a contiguous device tensor")
        self._keep = w   # emb is referenced by the handle
        self.dims = Dims(vocab, depths, hidden, emb_dim, state_dim, rank, max_batch, self.wdtype)
        self.wts = Weights(_ptr(w["emb"]), _ptr(w["w_ih"]), _ptr(w["w_hh"]), _ptr(w.get("b_ih")),
                           _ptr(w.get("b_hh")), _ptr(w["w1"]), _ptr(w["w2"]), _ptr(w.get("w_lm")))
        self.maxp = Params(max_top_m, max_top_k, max_budget, 1.0, DT_NORM_TOPM, 0)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self.handle = dt_create(self.dims, self.wts, self.maxp, self.stream.cuda_stream)

    def close(self):
        if getattr(self, "handle", None):
            dt_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def outputs(self, batch: int, top_m: int, budget: int, candidates: bool = False) -> dict:
        torch = self.torch
        dev = self._keep["w_ih"].device
        o = {
            "tokens": torch.empty((batch, budget + 1), dtype=torch.int32, device=dev),
            "parents": torch.empty((batch, budget + 1), dtype=torch.int32, device=dev),
            "depths": torch.empty((batch, budget + 1), dtype=torch.int32, device=dev),
            "scores": torch.empty((batch, budget + 1), dtype=torch.float32, device=dev),
            "n_nodes": torch.empty((batch,), dtype=torch.int32, device=dev),
        }
        if candidates:
            D = self.dims.depths
            o["cand_ids"] = torch.empty((batch, D, top_m), dtype=torch.int32, device=dev)
            o["cand_logits"] = torch.empty((batch, D, top_m), dtype=torch.float32, device=dev)
            o["lse"] = torch.empty((batch, D), dtype=torch.float32, device=dev)
        return o

    def build(self, hidden, base_logits=None, root_state=None, *, top_m, top_k, budget,
              temperature=1.0, norm=DT_NORM_TOPM, flags=None, out=None, candidates=False):
        """Enqueue one build on the builder's stream; returns the output tensors."""
        if flags is None:
            flags = DT_ACT_BF16 if self.wdtype == DT_BF16 else 0
        batch = hidden.shape[0]
        for name, t in (("hidden", hidden), ("base_logits", base_logits), ("root_state", root_state)):
            if t is not None and (not t.is_cuda or not t.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous device tensor")
        o = out if out is not None else self.outputs(batch, top_m, budget, candidates)
        inp = Inputs(batch, _ptr(base_logits), _ptr(hidden), _ptr(root_state))
        prm = Params(top_m, top_k, budget, float(temperature), norm, flags)
        outs = Outputs(_ptr(o["tokens"]), _ptr(o["parents"]), _ptr(o["depths"]), _ptr(o["scores"]),
                       _ptr(o["n_nodes"]), _ptr(o.get("cand_ids")), _ptr(o.get("cand_logits")),
                       _ptr(o.get("lse")))
        dt_build_trees(self.handle, inp, prm, outs, self.stream.cuda_stream)
        return o

    def chain(self, hidden, base_logits=None, root_state=None, *, flags=None, out=None):
        """Enqueue the greedy chain head (dt_draft_chain) on the builder's
        stream; returns {"tokens": [b, D] int32, "logits": [b, D] float32}."""
        torch = self.torch
        if flags is None:
            flags = DT_ACT_BF16 if self.wdtype == DT_BF16 else 0
        for name, t in (("hidden", hidden), ("base_logits", base_logits), ("root_state", root_state)):
            if t is not None and (not t.is_cuda or not t.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous device tensor")
        b, D = hidden.shape[0], self.dims.depths
        dev = self._keep["w_ih"].device
        o = out if out is not None else {
            "tokens": torch.empty((b, D), dtype=torch.int32, device=dev),
            "logits": torch.empty((b, D), dtype=torch.float32, device=dev)}
        inp = Inputs(b, _ptr(base_logits), _ptr(hidden), _ptr(root_state))
        dt_draft_chain(self.handle, inp, flags, _ptr(o["tokens"]), _ptr(o.get("logits")),
                       self.stream.cuda_stream)
        return o

    def fold_state(self, tokens, prev_state=None, *, flags=None, out=None):
        """S <- GRU(S, E[t]) over tokens [b, L] (int32 device tensor) from
        prev_state ([b, d_s] float32 or None = zeros); returns [b, d_s]."""
        torch = self.torch
        if flags is None:
            flags = DT_ACT_BF16 if self.wdtype == DT_BF16 else 0
        for name, t in (("tokens", tokens), ("prev_state", prev_state)):
            if t is not None and (not t.is_cuda or not t.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous device tensor")
        if tokens.dtype != torch.int32:
            raise ValueError("tokens must be int32")
        b, L = tokens.shape
        o = out if out is not None else torch.empty((b, self.dims.state_dim), dtype=torch.float32,
                                                    device=tokens.device)
        dt_fold_state(self.handle, b, L, _ptr(tokens), _ptr(prev_state), _ptr(o), flags,
                      self.stream.cuda_stream)
        return o

    def sync_status(self):
        dt_sync_status(self.handle, self.stream.cuda_stream)

    def phase_times(self) -> tuple:
        """Mean ms per phase (PHASES order: the LM head or P, candidates, the
        wait for P, builder set-up, tree kernel) of the DT_TIMING builds since
        the previous call, and how many builds were averaged."""
        return dt_phase_times(self.handle)


def tree_attention_inputs(parents, depths, n_nodes, tokens=None, prefix_len=None, anchor=None,
                          stream=None) -> dict:
    """Tree-attention inputs of built trees (torch int32 device tensors in the
    builder's output layout, [b, cols]).  Returns device tensors: mask
    [b, cols, ceil(cols / 32)] int32 (bit patterns of the uint32 words),
    positions [b, cols], tokens [b, cols] (when `tokens` is given) and bad [b]."""
    import torch
    b, cols = parents.shape
    for name, t in (("parents", parents), ("depths", depths), ("n_nodes", n_nodes),
                    ("tokens", tokens), ("prefix_len", prefix_len), ("anchor", anchor)):
        if t is not None and (not t.is_cuda or not t.is_contiguous() or t.dtype != torch.int32):
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    dev = parents.device
    words = (cols + 31) // 32
    o = {"mask": torch.empty((b, cols, words), dtype=torch.int32, device=dev),
         "positions": torch.empty((b, cols), dtype=torch.int32, device=dev),
         "bad": torch.empty((b,), dtype=torch.int32, device=dev)}
    if tokens is not None:
        o["tokens"] = torch.empty((b, cols), dtype=torch.int32, device=dev)
    view = TreeView(b, cols, _ptr(parents), _ptr(depths), _ptr(tokens), _ptr(n_nodes),
                    _ptr(prefix_len), _ptr(anchor))
    vo = VerifyOutputs(_ptr(o["mask"]), _ptr(o["positions"]), _ptr(o.get("tokens")), _ptr(o["bad"]))
    st = stream if stream is not None else torch.cuda.current_stream()
    dt_tree_attention_inputs(view, vo, st.cuda_stream)
    return o
