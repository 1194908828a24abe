#!/usr/bin/env python3
"""Throughput of the conditional best-first draft-tree builder on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload q8b_b32] [--cpu-seconds S]
                    [--no-cpu] [--no-lm-leg] [--copy-calibration MIB]

A step is one dt_build_trees call over one batch of synthetic inputs already
resident in HBM: per-depth top-M + LSE over the base logits, P = H W1_H, and
the persistent tree kernel (all requests of the batch, N nodes each).  Prints
one JSON line.  The default workload is the Qwen3-8B-shaped batch of 32
requests (V=151936, 15 depths, h=4096, d_s=1024, r=256, M=32, k=8, N=128,
T=0.5), with bf16 weights and fp32 accumulation.

The K timed steps carry no event records between their phases; a second pass
of K builds with DT_TIMING gives the per-phase HIP-event times (recorded on
the builder's stream, where the kernels run) and the tree kernel's mean
duration for its roofline.  With the default workload a second leg times the
LM-head pipeline (32 requests from hidden states through W_lm [4096, 151936],
M=64, k=8, N=256) for the LM-head GEMM's MFMA roofline.
"""
import argparse
import contextlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tree nodes/sec & µs/tree (batch 32, Qwen3-8B shape); % of HBM roofline"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def streaming_equivalent_bytes(spec) -> float:
    """Bytes a builder that streams the per-node weights would move per launch.

    Per step (one node expanded per request): W_ih, W_hh and the state half of
    W1 read once for the whole batch, plus per request the embedding row, the
    r x M slice of W2, P_d, the M base logits and the state read and written;
    N steps.  The builder here does not stream these weights (the input term
    is a per-token table, W_hh and W1_S stay in registers), so this volume
    divided by the kernel's time is a comparison with such a builder, not an
    HBM rate.
    """
    wb = 2 if spec.wdtype == "bf16" else 4
    per_step_weights = (3 * spec.ds * spec.e + 3 * spec.ds * spec.ds + spec.ds * spec.r) * wb
    per_request = spec.e * wb + spec.M * spec.r * wb + spec.r * 4 + spec.M * 4 + 2 * spec.ds * 4
    return float(spec.N) * (per_step_weights + spec.B * per_request)


def tree_kernel_per_node_bytes(spec) -> int:
    """HBM bytes one node's expansion must move in the builder as designed.

    The GRU input term of the node's token is a row of the per-token table
    G = E W_ih^T + b_ih (3 d_s fp32); the parent's gh = W_hh S + b_hh row
    (3 d_s fp32) and state (d_s fp32) are read; the node's state (d_s fp32)
    and its matrix-operand copy (d_s, weight dtype) are written; the workers
    write gh and u = W1_S^T S ((3 d_s + r) fp32) and the controller reads u
    back (r fp32).
    """
    wb = 2 if spec.wdtype == "bf16" else 4
    ds, r = spec.ds, spec.r
    return 3 * ds * 4 + 3 * ds * 4 + ds * 4 + ds * 4 + ds * wb + (3 * ds + r) * 4 + r * 4


def tree_kernel_fixed_bytes(spec) -> int:
    """HBM bytes a launch moves once: the per-node weights [W_hh; W1_S^T]
    loaded into the workers, each request's W2 candidate rows (D depths x M x
    r), P, the candidate tables and tails, and the outputs."""
    wb = 2 if spec.wdtype == "bf16" else 4
    ds, r, B, D, M = spec.ds, spec.r, spec.B, spec.D, spec.M
    weights = (3 * ds + r) * ds * wb
    w2rows = B * D * M * r * wb
    p = B * D * r * 4
    cands = B * D * M * 12 + B * D * 4
    outs = B * (spec.N + 1) * 16 + B * 4
    return weights + w2rows + p + cands + outs


def tree_kernel_bytes(spec) -> float:
    """Algorithmic HBM bytes of one tree-kernel launch: B N nodes, each
    expanded once, plus the launch's fixed bytes."""
    return float(spec.B * spec.N * tree_kernel_per_node_bytes(spec) + tree_kernel_fixed_bytes(spec))


def tree_kernel_flops(spec, nodes: float) -> float:
    """Matrix-core flops of the per-node products [W_hh; W1_S^T] S for `nodes`
    expanded nodes."""
    return 2.0 * nodes * (3 * spec.ds + spec.r) * spec.ds


TREE_SOURCES = ["csrc/tree.hip", "csrc/tree.h", "csrc/common.h", "csrc/kernels.h"]


def tree_source_hash() -> str:
    """sha256 of the sources the tree kernel is compiled from."""
    import hashlib
    h = hashlib.sha256()
    for f in TREE_SOURCES:
        with open(os.path.join(ROOT, "conditional_draft_tree_dominotree_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per tree-kernel launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size),
    or None when there is none or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_tree_kernel_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("tree_source_sha256") != tree_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def to_dev(a):
    """A numpy array (bf16 stored as uint16 bits) as a contiguous device tensor."""
    import numpy as np
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def _oracle_run(spec, w, req, seconds: float, threads):
    """The CPU oracle on the first requests of the workload, for about
    `seconds` of wall time, with BLAS limited to `threads` (None: as set)."""
    from oracle import ref
    limit = contextlib.nullcontext()
    if threads is not None:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=threads, user_api="blas")
    bf16 = spec.wdtype == "bf16"
    head = ref.make_head(w, bf16, spec.act_bf16)
    done, nodes, trees = 0, 0, []
    with limit:
        used = blas_threads()
        t0 = time.perf_counter()
        while done < spec.B:
            hid = ref.hidden_values(req["hidden"][done], bf16)
            if req["base"] is not None:
                base = req["base"][done]
            else:  # the LM-head workload: the oracle computes the base logits too
                base = ref.lm_head_logits(req["hidden"][done], w["w_lm"], bf16)
            t = ref.build_tree(head, base, hid, req["root"][done], spec.M, spec.k, spec.N, spec.T,
                               spec.norm)
            trees.append(t)
            nodes += t.n_nodes
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        el = time.perf_counter() - t0
    return {"value": nodes / el, "us_per_tree": el / done * 1e6, "cores": used,
            "sample": f"first {done} of {spec.B} requests of {spec.name} ({nodes} nodes), {el:.1f} s wall"}, trees


def cpu_baseline(spec, w, req, seconds: float):
    """The oracle (NumPy float64, a heapq best-first loop per request) timed
    on the host: once with BLAS on every core it is given, once on one thread.
    Returns the baseline object and the all-cores run's trees."""
    allc, trees = _oracle_run(spec, w, req, seconds, None)
    one, _ = _oracle_run(spec, w, req, seconds, 1)
    res = {
        "value": allc["value"],
        "unit": "nodes/s",
        "cores": allc["cores"],
        "kind": "oracle",
        "sample": allc["sample"] + "; NumPy float64 heapq builder, BLAS threads = cores",
        "us_per_tree": allc["us_per_tree"],
        "one_thread": {"value": one["value"], "unit": "nodes/s", "cores": 1, "us_per_tree": one["us_per_tree"],
                       "sample": one["sample"]},
        "host": {"os_cpu_count": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0))},
    }
    return res, trees


def lm_head_leg(steps: int, warmup: int) -> dict:
    """The LM-head pipeline (hidden states -> W_lm -> candidates -> tree) at
    32 requests: its round time and the LM-head GEMM's MFMA roofline."""
    import numpy as np
    import torch

    import conditional_draft_tree_dominotree_amd as pkg
    from workloads import synth
    spec, w, req = synth.workload("q8b_lm")
    wdev = {k: to_dev(v) for k, v in w.items()}
    tb = pkg.TreeBuilder(wdev, vocab=spec.V, depths=spec.D, hidden=spec.h, emb_dim=spec.e,
                         state_dim=spec.ds, rank=spec.r, max_batch=spec.B, max_top_m=spec.M,
                         max_top_k=spec.k, max_budget=spec.N)
    hidden = to_dev(req["hidden"])
    out = tb.outputs(spec.B, spec.M, spec.N)

    def step(extra=0):
        tb.build(hidden, None, None, top_m=spec.M, top_k=spec.k, budget=spec.N, temperature=spec.T,
                 flags=pkg.DT_ACT_BF16 | extra, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    tb.sync_status()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(tb.stream)
    for _ in range(steps):
        step()
    e1.record(tb.stream)
    torch.cuda.synchronize()
    round_ms = e0.elapsed_time(e1) / steps
    tb.phase_times()
    for _ in range(steps):
        step(pkg.DT_TIMING)
    torch.cuda.synchronize()
    tb.sync_status()
    phases, nb = tb.phase_times()
    assert np.all(out["n_nodes"].cpu().numpy() == spec.N)
    tb.close()
    del wdev, hidden, out
    torch.cuda.empty_cache()
    flops = 2.0 * spec.B * spec.D * spec.V * spec.h
    tf = flops / (phases[0] * 1e-3) / 1e12
    return {
        "workload": f"{spec.name}: B={spec.B}, H [{spec.B * spec.D}, {spec.h}] bf16 x W_lm [{spec.h}, {spec.V}] "
                    f"bf16 (fp32 accumulation), then M={spec.M}, k={spec.k}, N={spec.N}, T={spec.T}",
        "round_ms": round_ms,
        "nodes_per_s": spec.B * spec.N / (round_ms * 1e-3),
        "phases_ms": {"lm_head": phases[0], "candidates": phases[1], "P_join": phases[2],
                      "builder_setup": phases[3], "tree_kernel": phases[4], "builds_averaged": nb},
        "roofline": {"kernel": "gemm_lm_topk_kernel (H W_lm with the per-list top-8 and LSE epilogue; the "
                                "per-call re-layout of H included)", "bound": "mfma",
                     "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS,
                     "traffic": None, "algorithmic_flops": flops},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="q8b_b32")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-lm-leg", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed run, copy a MIB-MiB buffer 3 times (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the builder has no multi-GPU path (requests shard "
              "independently; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import conditional_draft_tree_dominotree_amd as pkg
    from workloads import synth

    pkg.load_library()   # fails loudly when the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    spec, w, req = synth.workload(args.workload)
    wdev = {k: to_dev(v) for k, v in w.items()}
    torch.cuda.synchronize()
    tc0 = time.perf_counter()
    tb = pkg.TreeBuilder(wdev, vocab=spec.V, depths=spec.D,
                         hidden=spec.h, emb_dim=spec.e, state_dim=spec.ds, rank=spec.r,
                         max_batch=spec.B, max_top_m=spec.M, max_top_k=spec.k, max_budget=spec.N)
    torch.cuda.synchronize()
    create_s = time.perf_counter() - tc0   # tables and prepack, once per weight set
    hidden = to_dev(req["hidden"])
    base = to_dev(req["base"]) if req["base"] is not None else None
    norm = pkg.DT_NORM_FULLV if spec.norm == "fullv" else pkg.DT_NORM_TOPM
    flags = pkg.DT_ACT_BF16 if spec.wdtype == "bf16" else 0
    out = tb.outputs(spec.B, spec.M, spec.N, stats=True)

    def step(extra=0):
        tb.build(hidden, base, None, top_m=spec.M, top_k=spec.k, budget=spec.N,
                 temperature=spec.T, norm=norm, flags=flags | extra, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    tb.sync_status()
    tb.phase_times()   # start a fresh averaging window
    stream = tb.stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tb.sync_status()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    # per-phase HIP events (DT_TIMING) in a second pass of the same builds,
    # so that the timed pass carries no event records between the phases
    for _ in range(args.steps):
        step(pkg.DT_TIMING)
    torch.cuda.synchronize()
    tb.sync_status()
    phases, nb = tb.phase_times()
    stats = out["stats"].cpu().numpy()
    # round-time distribution: ROUNDS builds one by one with events around
    # each, warm (nothing in between) and cold (a 512 MB buffer written
    # between builds, which evicts the caches: MALL and L2); the buffer
    # write doubles as a measure of the box's achievable HBM bandwidth
    ROUNDS = 50
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    dist = {}
    for mode in ("warm", "cold"):
        ts = []
        for _ in range(ROUNDS):
            if mode == "cold":
                scratch.fill_(1)
            r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            r0.record(stream)
            step()
            r1.record(stream)
            torch.cuda.synchronize()
            ts.append(r0.elapsed_time(r1))
        ts = np.array(ts)
        dist[mode] = {"median_ms": float(np.median(ts)), "p10_ms": float(np.percentile(ts, 10)),
                      "p90_ms": float(np.percentile(ts, 90))}
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    for _ in range(10):
        scratch.fill_(2)
    f1.record()
    torch.cuda.synchronize()
    fill_gbs = 10 * scratch.numel() / (f0.elapsed_time(f1) * 1e-3) / 1e9
    del scratch
    tb.sync_status()
    # the verification inputs of the built trees (ancestor mask, positions,
    # flattened tokens), timed on the builder's stream beside the build
    prefix = torch.zeros(spec.B, dtype=torch.int32, device="cuda")
    anchor = torch.zeros(spec.B, dtype=torch.int32, device="cuda")
    vo = pkg.tree_attention_inputs(out["parents"], out["depths"], out["n_nodes"], tokens=out["tokens"],
                                   prefix_len=prefix, anchor=anchor, stream=stream)
    from conditional_draft_tree_dominotree_amd import binding
    view = binding.TreeView(spec.B, spec.N + 1, out["parents"].data_ptr(), out["depths"].data_ptr(),
                            out["tokens"].data_ptr(), out["n_nodes"].data_ptr(), prefix.data_ptr(),
                            anchor.data_ptr())
    vouts = binding.VerifyOutputs(vo["mask"].data_ptr(), vo["positions"].data_ptr(), vo["tokens"].data_ptr(),
                                  vo["bad"].data_ptr())
    v0, v1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    v0.record(stream)
    for _ in range(args.steps):
        binding.dt_tree_attention_inputs(view, vouts, stream.cuda_stream)
    v1.record(stream)
    torch.cuda.synchronize()
    assert int(vo["bad"].sum().item()) == 0
    verify_ms = v0.elapsed_time(v1) / args.steps
    # the greedy chain head over the whole vocabulary on the same weights and
    # inputs, for the whole batch and for its first request alone
    chain_ms = {}
    for cb in ((spec.B, 1) if spec.B > 1 else (1,)):
        hid_b = hidden[:cb].contiguous()
        base_b = base[:cb].contiguous() if base is not None else None
        co = tb.chain(hid_b, base_b)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(args.steps):
            tb.chain(hid_b, base_b, out=co)
        c1.record(stream)
        torch.cuda.synchronize()
        tb.sync_status()
        chain_ms[f"batch_{cb}"] = c0.elapsed_time(c1) / args.steps
    # the sampled chain (Gumbel-max at T = 1) for the whole batch
    co = tb.chain(hidden, base, temperature=1.0, seed=1)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for i in range(args.steps):
        tb.chain(hidden, base, out=co, temperature=1.0, seed=2 + i)
    c1.record(stream)
    torch.cuda.synchronize()
    tb.sync_status()
    chain_ms[f"sampled_batch_{spec.B}"] = c0.elapsed_time(c1) / args.steps

    def timed_rounds(extra=0):
        for _ in range(2):
            step(extra)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(args.steps):
            step(extra)
        a1.record(stream)
        torch.cuda.synchronize()
        tb.sync_status()
        return a0.elapsed_time(a1) / args.steps

    # ablations on the same builds (event time per round): the factorised
    # tree (DT_MARGINAL: base logits alone, no per-node products), a
    # cooperative instead of a plain launch, the correction dL with vector FMAs,
    # the workers' group exchange device-wide instead of through their XCD's L2
    ablations = {"marginal_round_ms": timed_rounds(pkg.DT_MARGINAL)}
    for key, sched in (("cooperative_launch_round_ms", dict(launch=2)), ("fma_dl_round_ms", dict(dl=1)),
                       ("device_exchange_round_ms", dict(exchange=1))):
        tb.set_schedule(**sched)
        ablations[key] = timed_rounds()
        tb.set_schedule()
    step()
    torch.cuda.synchronize()
    tb.sync_status()
    n_nodes = out["n_nodes"].cpu().numpy()
    assert np.all(n_nodes == spec.N), n_nodes

    nodes = spec.B * spec.N
    value = nodes / (wall_ms * 1e-3)
    tree_ms = phases[4]
    ab = tree_kernel_bytes(spec)
    achieved = ab / (tree_ms * 1e-3) / 1e9
    traffic = measured_traffic(spec.name)
    expanded = float(stats[:, 1].sum())
    flops_alg = tree_kernel_flops(spec, nodes)
    flops_done = tree_kernel_flops(spec, expanded)
    steps_max = int(stats[:, 0].max())
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.wdtype,
        "data": "synthetic",
        "config": {
            "workload": f"{spec.name}: B={spec.B} requests, V={spec.V}, D={spec.D} depths, "
                        f"h={spec.h}, e={spec.e}, d_s={spec.ds}, r={spec.r}, M={spec.M}, "
                        f"k={spec.k}, N={spec.N}, T={spec.T}, norm={spec.norm}, "
                        f"weights {spec.wdtype} with fp32 accumulation",
            "global_batch": spec.B,
        },
        "us_per_tree": wall_ms * 1e3 / spec.B,
        "round_ms_events": ev_ms,
        "ablations": ablations,
        "phases_ms": {"lm_head_or_P": phases[0], "candidates": phases[1], "P_join": phases[2],
                      "builder_setup": phases[3], "tree_kernel": tree_ms, "builds_averaged": nb},
        "round_ms_distribution": dict(dist, rounds=ROUNDS),
        "handle_create_s": create_s,
        "hbm_write_gbs_measured": fill_gbs,
        "chain_head_ms": dict(chain_ms, positions=spec.D, launch="dt_draft_chain (greedy, full vocabulary)"),
        "verify_inputs": {"ms": verify_ms, "launch": "dt_tree_attention_inputs",
                          "bytes": spec.B * (spec.N + 1) * 4 * (5 + (spec.N + 32) // 32) + spec.B * 12},
        # the dominant kernel: HBM bytes the builder as designed must move
        # (B N node expansions plus the launch's fixed loads) over its mean
        # event duration
        "roofline": {
            "kernel": "tree_kernel",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes": ab,
            "units": f"{nodes} node expansions x {tree_kernel_per_node_bytes(spec)} B + "
                     f"{tree_kernel_fixed_bytes(spec)} B per launch",
            "traffic_frac": None if traffic is None else traffic / (tree_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma": {"flops_algorithmic": flops_alg, "flops_done": flops_done,
                     "frac": flops_done / (tree_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                     "what": "[W_hh; W1_S^T] S products of the expanded nodes (speculative ones included)"},
            "latency": {"steps_max": steps_max, "steps_mean": float(stats[:, 0].mean()),
                        "us_per_step": tree_ms * 1e3 / steps_max,
                        "expansions_per_request": float(stats[:, 1].mean()), "nodes_per_request": spec.N},
            "streaming_equivalent": {
                "bytes": streaming_equivalent_bytes(spec),
                "gbs": streaming_equivalent_bytes(spec) / (tree_ms * 1e-3) / 1e9,
                "what": "the per-node weights streamed once per step for the batch, over the tree kernel's time "
                        "(a comparison with a streaming builder, not an HBM rate)"},
        },
    }
    if base is None:
        # the LM head: a dense bf16 contraction, priced against the MFMA peak
        flops = 2.0 * spec.B * spec.D * spec.V * spec.h
        tf = flops / (phases[0] * 1e-3) / 1e12
        res["roofline_lm_head"] = {"kernel": "gemm_lm_topk_kernel (H W_lm with the candidate epilogue)",
                                   "bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                   "frac": tf / BF16_PEAK_TFLOPS, "traffic": None,
                                   "algorithmic_flops": flops}
    got = {k: v.cpu().numpy() for k, v in out.items()}
    tb.close()
    del wdev, hidden, base, out
    torch.cuda.empty_cache()
    if args.workload == "q8b_b32" and not args.no_lm_leg:
        leg = lm_head_leg(max(5, args.steps // 2), args.warmup)
        res["lm_head_leg"] = leg
        res["roofline_lm_head"] = leg["roofline"]
    if not args.no_cpu:
        # CPU-baseline leg: the oracle, timed on a bounded sample of the workload
        from oracle import certify, ref
        cb, trees = cpu_baseline(spec, w, req, args.cpu_seconds)
        res["cpu_baseline"] = cb
        # the sample's trees double as a parity spot check of the timed output
        head = ref.make_head(w, spec.wdtype == "bf16", spec.act_bf16)
        tol = 2e-2 if spec.wdtype == "bf16" else 1e-4
        reps = []
        for b, t in enumerate(trees):
            other = {k: got[k][b] for k in ("tokens", "parents", "depths", "scores")}
            other["n_nodes"] = int(got["n_nodes"][b])
            hid = ref.hidden_values(req["hidden"][b], spec.wdtype == "bf16")
            reps.append(certify.compare(t, head, hid, req["root"][b], other, spec.k, spec.T,
                                        spec.norm, spec.N, tol))
        census = {}
        for r in reps:
            for key, v in r.census.items():
                census[key] = census.get(key, 0) + v
        res["parity_sample"] = {"requests": len(reps), "exact": sum(r.exact for r in reps),
                                "ok": all(r.ok for r in reps),
                                "near_ties": [r.near_tie for r in reps if not r.exact],
                                "max_abs_dscore": max(r.max_dscore for r in reps),
                                "tol": tol, "decisions_within_tol": census,
                                "trees_with_no_decision_within_tol": sum(r.must_be_exact for r in reps)}
    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = n * 4
    print(json.dumps(res))


if __name__ == "__main__":
    main()
