"""ctypes binding of libdominotree.so (argument marshalling only).

The dt_* functions mirror include/dominotree.h one to one; TreeBuilder and
tree_attention_inputs wrap them for torch device tensors and check every
tensor's device, dtype, shape and layout against the handle's dimensions
before a pointer reaches the library (a wrong size would make a kernel read
past an allocation).  Every step of the build runs in the HIP library: when
it is not built, loading fails loudly.
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
                ("cand_logits", C.c_void_p), ("lse", C.c_void_p), ("stats", C.c_void_p),
                ("logits", C.c_void_p)]


class Schedule(C.Structure):
    _fields_ = [("pops", C.c_int32), ("halves", C.c_int32), ("lds_workers", C.c_int32),
                ("tiles_per_worker", C.c_int32), ("advance", C.c_int32), ("launch", C.c_int32),
                ("dl", C.c_int32), ("exchange", C.c_int32)]


class TreeView(C.Structure):
    _fields_ = [("batch", C.c_int32), ("cols", C.c_int32), ("parents", C.c_void_p),
                ("depths", C.c_void_p), ("tokens", C.c_void_p), ("n_nodes", C.c_void_p),
                ("prefix_len", C.c_void_p), ("anchor", C.c_void_p)]


class VerifyOutputs(C.Structure):
    _fields_ = [("mask", C.c_void_p), ("positions", C.c_void_p), ("tokens", C.c_void_p),
                ("bad", C.c_void_p)]


EXPORTS = ["dt_create", "dt_build_trees", "dt_sync_status", "dt_phase_times", "dt_destroy",
           "dt_last_error", "dt_version", "dt_tree_attention_inputs", "dt_draft_chain", "dt_fold_state",
           "dt_set_schedule", "dt_set_device_error", "dt_draft_chain_noalloc", "dt_draft_chain_sample"]
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
    lib.dt_draft_chain_sample.restype = C.c_int
    lib.dt_draft_chain_sample.argtypes = [C.c_void_p, C.POINTER(Inputs), C.c_uint32, C.c_float, C.c_uint64,
                                          C.c_void_p, C.c_void_p, C.c_void_p]
    lib.dt_draft_chain_noalloc.restype = C.c_int
    lib.dt_draft_chain_noalloc.argtypes = [C.c_void_p, C.POINTER(Inputs), C.c_uint32, C.c_void_p, C.c_void_p,
                                           C.c_void_p]
    lib.dt_fold_state.restype = C.c_int
    lib.dt_fold_state.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_uint32, C.c_void_p]
    lib.dt_set_schedule.restype = C.c_int
    lib.dt_set_schedule.argtypes = [C.c_void_p, C.POINTER(Schedule)]
    lib.dt_set_device_error.restype = C.c_int
    lib.dt_set_device_error.argtypes = [C.c_void_p, C.c_int32, C.c_void_p]
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


def dt_draft_chain_sample(handle: int, inputs: Inputs, flags: int, temperature: float, seed: int, tokens: int,
                          logits, stream: int = 0):
    _check(load_library().dt_draft_chain_sample(C.c_void_p(handle), C.byref(inputs), C.c_uint32(flags),
                                                C.c_float(temperature), C.c_uint64(seed), C.c_void_p(tokens),
                                                C.c_void_p(logits), C.c_void_p(stream)))


def dt_draft_chain_noalloc(handle: int, inputs: Inputs, flags: int, tokens: int, logits, stream: int = 0):
    _check(load_library().dt_draft_chain_noalloc(C.c_void_p(handle), C.byref(inputs), C.c_uint32(flags),
                                                 C.c_void_p(tokens), C.c_void_p(logits), C.c_void_p(stream)))


def dt_fold_state(handle: int, batch: int, n_tokens: int, tokens: int, prev_state, state_out: int,
                  flags: int, stream: int = 0):
    _check(load_library().dt_fold_state(C.c_void_p(handle), batch, n_tokens, C.c_void_p(tokens),
                                        C.c_void_p(prev_state), C.c_void_p(state_out), C.c_uint32(flags),
                                        C.c_void_p(stream)))


def dt_set_schedule(handle: int, sched):
    """sched: a Schedule, or None for the defaults."""
    _check(load_library().dt_set_schedule(C.c_void_p(handle), None if sched is None else C.byref(sched)))


def dt_set_device_error(handle: int, code: int, stream: int = 0):
    _check(load_library().dt_set_device_error(C.c_void_p(handle), code, C.c_void_p(stream)))


def dt_tree_attention_inputs(view: TreeView, out: VerifyOutputs, stream: int = 0):
    _check(load_library().dt_tree_attention_inputs(C.byref(view), C.byref(out), C.c_void_p(stream)))


# ----------------------------------------------------------------------------
# torch convenience layer


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, dtype, shape, device=None, optional=False, where=True):
    """Refuse a tensor whose dtype, shape, layout or (with `where`) device the
    library would misread (ValueError, before any pointer reaches the C ABI)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not where:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the handle on {device}")


class TreeBuilder:
    """A handle plus caller-owned output tensors, for torch device tensors.

    weights: dict with emb [V, e], w_ih [3 d_s, e], w_hh [3 d_s, d_s],
    w1 [h + d_s, r], w2 [r, V] (all torch.float32, or all torch.bfloat16),
    optional b_ih, b_hh ([3 d_s] float32) and w_lm ([h, V], bf16); contiguous,
    on one device.
    """

    def __init__(self, weights: dict, *, vocab, depths, hidden, emb_dim, state_dim, rank,
                 max_batch, max_top_m, max_top_k, max_budget, stream=None):
        import torch
        self.torch = torch
        w = {k: v for k, v in weights.items() if v is not None}
        for k in ("emb", "w_ih", "w_hh", "w1", "w2"):
            if k not in w:
                raise ValueError(f"weight {k} is required")
        dt = w["w_ih"].dtype
        if dt not in (torch.float32, torch.bfloat16):
            raise ValueError(f"weights must be float32 or bfloat16, got {dt}")
        self.wdtype = DT_BF16 if dt == torch.bfloat16 else DT_F32
        self.tdtype = dt
        dev = w["w_ih"].device
        V, h, e, ds, r = vocab, hidden, emb_dim, state_dim, rank
        shapes = {"emb": (V, e), "w_ih": (3 * ds, e), "w_hh": (3 * ds, ds), "w1": (h + ds, r),
                  "w2": (r, V), "w_lm": (h, V)}
        for where in (False, True):   # every dtype and shape first, then the devices
            for k, shp in shapes.items():
                _check_tensor(f"weight {k}", w.get(k), dt, shp, dev, optional=k == "w_lm", where=where)
            for k in ("b_ih", "b_hh"):
                _check_tensor(f"weight {k}", w.get(k), torch.float32, (3 * ds,), dev, optional=True,
                              where=where)
        self.device = dev
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

    def outputs(self, batch: int, top_m: int, budget: int, candidates: bool = False,
                stats: bool = False, logits: bool = False) -> dict:
        torch = self.torch
        dev = self.device
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
        if stats:
            o["stats"] = torch.empty((batch, 2), dtype=torch.int32, device=dev)
        if logits:
            o["logits"] = torch.empty((batch, self.dims.depths, self.dims.vocab), dtype=torch.float32, device=dev)
        return o

    def _check_inputs(self, hidden, base_logits, root_state):
        torch = self.torch
        d = self.dims
        if hidden is None or hidden.dim() != 3:
            raise ValueError("hidden must be [batch, depths, hidden]")
        b = hidden.shape[0]
        if not 1 <= b <= d.max_batch:
            raise ValueError(f"batch {b} outside 1..{d.max_batch}")
        for where in (False, True):
            _check_tensor("hidden", hidden, self.tdtype, (b, d.depths, d.hidden), self.device, where=where)
            _check_tensor("base_logits", base_logits, torch.float32, (b, d.depths, d.vocab), self.device,
                          optional=True, where=where)
            _check_tensor("root_state", root_state, torch.float32, (b, d.state_dim), self.device,
                          optional=True, where=where)
        return b

    def build(self, hidden, base_logits=None, root_state=None, *, top_m, top_k, budget,
              temperature=1.0, norm=DT_NORM_TOPM, flags=None, out=None, candidates=False):
        """Enqueue one build on the builder's stream; returns the output tensors."""
        torch = self.torch
        if flags is None:
            flags = DT_ACT_BF16 if self.wdtype == DT_BF16 else 0
        batch = self._check_inputs(hidden, base_logits, root_state)
        o = out if out is not None else self.outputs(batch, top_m, budget, candidates)
        for k in ("tokens", "parents", "depths"):
            _check_tensor(f"output {k}", o.get(k), torch.int32, (batch, budget + 1), self.device)
        _check_tensor("output scores", o.get("scores"), torch.float32, (batch, budget + 1), self.device)
        _check_tensor("output n_nodes", o.get("n_nodes"), torch.int32, (batch,), self.device)
        D = self.dims.depths
        _check_tensor("output cand_ids", o.get("cand_ids"), torch.int32, (batch, D, top_m), self.device,
                      optional=True)
        _check_tensor("output cand_logits", o.get("cand_logits"), torch.float32, (batch, D, top_m),
                      self.device, optional=True)
        _check_tensor("output lse", o.get("lse"), torch.float32, (batch, D), self.device, optional=True)
        _check_tensor("output stats", o.get("stats"), torch.int32, (batch, 2), self.device, optional=True)
        _check_tensor("output logits", o.get("logits"), torch.float32, (batch, D, self.dims.vocab), self.device,
                      optional=True)
        inp = Inputs(batch, _ptr(base_logits), _ptr(hidden), _ptr(root_state))
        prm = Params(top_m, top_k, budget, float(temperature), norm, flags)
        outs = Outputs(_ptr(o["tokens"]), _ptr(o["parents"]), _ptr(o["depths"]), _ptr(o["scores"]),
                       _ptr(o["n_nodes"]), _ptr(o.get("cand_ids")), _ptr(o.get("cand_logits")),
                       _ptr(o.get("lse")), _ptr(o.get("stats")), _ptr(o.get("logits")))
        dt_build_trees(self.handle, inp, prm, outs, self.stream.cuda_stream)
        return o

    def chain(self, hidden, base_logits=None, root_state=None, *, flags=None, out=None, temperature=None,
              seed=0):
        """Enqueue the chain head on the builder's stream: greedy
        (dt_draft_chain) when temperature is None, else sampled at that
        temperature with the given seed (dt_draft_chain_sample); returns
        {"tokens": [b, D] int32, "logits": [b, D] float32}."""
        torch = self.torch
        if flags is None:
            flags = DT_ACT_BF16 if self.wdtype == DT_BF16 else 0
        b = self._check_inputs(hidden, base_logits, root_state)
        D = self.dims.depths
        o = out if out is not None else {
            "tokens": torch.empty((b, D), dtype=torch.int32, device=self.device),
            "logits": torch.empty((b, D), dtype=torch.float32, device=self.device)}
        _check_tensor("output tokens", o.get("tokens"), torch.int32, (b, D), self.device)
        _check_tensor("output logits", o.get("logits"), torch.float32, (b, D), self.device, optional=True)
        inp = Inputs(b, _ptr(base_logits), _ptr(hidden), _ptr(root_state))
        if temperature is None:
            dt_draft_chain(self.handle, inp, flags, _ptr(o["tokens"]), _ptr(o.get("logits")),
                           self.stream.cuda_stream)
        else:
            dt_draft_chain_sample(self.handle, inp, flags, float(temperature), int(seed), _ptr(o["tokens"]),
                                  _ptr(o.get("logits")), self.stream.cuda_stream)
        return o

    def fold_state(self, tokens, prev_state=None, *, flags=None, out=None):
        """S <- GRU(S, E[t]) over tokens [b, L] (int32 device tensor) from
        prev_state ([b, d_s] float32 or None = zeros); returns [b, d_s]."""
        torch = self.torch
        if flags is None:
            flags = DT_ACT_BF16 if self.wdtype == DT_BF16 else 0
        if tokens is None or tokens.dim() != 2:
            raise ValueError("tokens must be [batch, n_tokens]")
        b, L = tokens.shape
        if not 1 <= b <= self.dims.max_batch:
            raise ValueError(f"batch {b} outside 1..{self.dims.max_batch}")
        ds = self.dims.state_dim
        for where in (False, True):
            _check_tensor("tokens", tokens, torch.int32, (b, L), self.device, where=where)
            _check_tensor("prev_state", prev_state, torch.float32, (b, ds), self.device, optional=True,
                          where=where)
        o = out if out is not None else torch.empty((b, ds), dtype=torch.float32, device=self.device)
        _check_tensor("state_out", o, torch.float32, (b, ds), self.device)
        dt_fold_state(self.handle, b, L, _ptr(tokens), _ptr(prev_state), _ptr(o), flags,
                      self.stream.cuda_stream)
        return o

    def sync_status(self):
        dt_sync_status(self.handle, self.stream.cuda_stream)

    def set_schedule(self, pops=0, halves=0, lds_workers=0, tiles_per_worker=0, advance=0, launch=0, dl=0,
                     exchange=0):
        """Schedule of the next builds (dt_set_schedule); all zeros: defaults."""
        dt_set_schedule(self.handle, Schedule(pops, halves, lds_workers, tiles_per_worker, advance, launch, dl,
                                              exchange))

    def set_device_error(self, code=1):
        """Test hook of the failure path (dt_set_device_error)."""
        dt_set_device_error(self.handle, code, self.stream.cuda_stream)

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
    if parents is None or parents.dim() != 2:
        raise ValueError("parents must be [batch, cols]")
    b, cols = parents.shape
    dev = parents.device
    for where in (False, True):
        for name, t, shp, opt in (("parents", parents, (b, cols), False), ("depths", depths, (b, cols), False),
                                  ("n_nodes", n_nodes, (b,), False), ("tokens", tokens, (b, cols), True),
                                  ("prefix_len", prefix_len, (b,), True), ("anchor", anchor, (b,), True)):
            _check_tensor(name, t, torch.int32, shp, dev, optional=opt, where=where)
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
