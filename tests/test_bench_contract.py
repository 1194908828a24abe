"""CPU checks of the measurement script's own arithmetic and contract (the
timed run itself needs a GPU)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import synth  # noqa: E402


def test_streaming_equivalent_bytes():
    # per step: W_ih + W_hh + the state half of W1 read once for the batch,
    # plus per request the embedding row, the r x M slice of W2, P_d, the M
    # base logits and the state read and written; N steps
    spec = synth.SPECS["q8b_b32"]
    per_step = (3 * 1024 * 4096 + 3 * 1024 * 1024 + 1024 * 256) * 2
    per_req = 4096 * 2 + 32 * 256 * 2 + 256 * 4 + 32 * 4 + 2 * 1024 * 4
    assert per_step == 31_981_568
    assert bench.streaming_equivalent_bytes(spec) == 128 * (per_step + 32 * per_req)
    assert abs(bench.streaming_equivalent_bytes(spec) - 4.2326e9) < 1e6


def test_tree_kernel_bytes_of_the_design():
    # per node: G row, parent's gh and state read; state, operand copy, gh and
    # u written; u read back (d_s = 1024, r = 256, bf16 operand copy)
    spec = synth.SPECS["q8b_b32"]
    per_node = 3 * 1024 * 4 * 2 + 1024 * 4 * 2 + 1024 * 2 + (3 * 1024 + 256) * 4 + 256 * 4
    assert bench.tree_kernel_per_node_bytes(spec) == per_node == 49_152
    fixed = (3 * 1024 + 256) * 1024 * 2 + 32 * 15 * 32 * 256 * 2 + 32 * 15 * 256 * 4 \
        + 32 * 15 * 32 * 12 + 32 * 15 * 4 + 32 * 129 * 16 + 32 * 4
    assert bench.tree_kernel_fixed_bytes(spec) == fixed
    assert bench.tree_kernel_bytes(spec) == 32 * 128 * per_node + fixed
    # far below the streaming-equivalent volume: the design reads no weights per step
    assert bench.tree_kernel_bytes(spec) < 0.06 * bench.streaming_equivalent_bytes(spec)
    assert bench.tree_kernel_flops(spec, 1) == 2 * (3 * 1024 + 256) * 1024


def test_traffic_figure_tracks_the_kernel_sources():
    # the committed counter summary is used only while its hash matches the
    # tree kernel's sources
    t = bench.measured_traffic("q8b_b32")
    assert t is None or 1e8 < t < 1e9
    assert bench.measured_traffic("no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
