"""Code-generation guards for the tree kernel (CPU: hipcc cross-compiles gfx950).

The builder's step time is dominated by memory round trips, so two properties
of the generated code matter as much as its arithmetic:
  * no private (scratch) memory, and
  * the worker's operand staging keeps its batch of 16-byte loads in flight
    together (a schedule that waits after each load multiplies the staging
    time by the batch size).
Both depend on register pressure across the whole kernel, so any edit can flip
them; these tests catch that without a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TREE = os.path.join(ROOT, "conditional_draft_tree_dominotree_amd", "csrc", "tree.hip")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("codegen") / "tree.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", "-o", str(out), TREE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernel(asm_text, tmpl):
    name = f"_ZN2dt11tree_kernelI{tmpl}EEvNS_8TreeArgsE"
    lines = asm_text.split("\n")
    start = next(i for i, l in enumerate(lines) if l.startswith(name + ":"))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    meta = re.search(re.escape(name) + r"\.private_seg_size, (\d+)", asm_text)
    return [l.strip() for l in lines[start:end]], (int(meta.group(1)) if meta else None)


@pytest.mark.parametrize("tmpl", ["t", "f"])  # bf16 and fp32 weights
def test_tree_kernel_uses_no_scratch(asm, tmpl):
    body, priv = _kernel(asm, tmpl)
    assert not any(l.startswith(("scratch_", "buffer_store_dword", "buffer_load_dword")) for l in body)
    if priv is not None:
        assert priv == 0


def _worker_region(body):
    # from the worker's mailbox poll (the sleep before the first MFMA) to the
    # last MFMA (only workers multiply on the matrix cores)
    mfma = [i for i, l in enumerate(body) if l.startswith("v_mfma")]
    poll = max(i for i, l in enumerate(body[:mfma[0]]) if l.startswith("s_sleep"))
    return body[poll:mfma[-1] + 1]


def _load_runs(body):
    # runs of 16-byte loads issued between two waits on vector memory
    runs, cur = [], []
    for l in _worker_region(body):
        if l.startswith("global_load_dwordx4"):
            cur.append(l)
        elif l.startswith("s_waitcnt") and "vmcnt" in l:
            if cur:
                runs.append(cur)
            cur = []
    return runs


def test_lds_worker_staging_loads_are_batched(asm):
    # the LDS worker's staging batch: 16 loads addressed from one base (saddr)
    runs = [r for r in _load_runs(_kernel(asm, "t")[0]) if all(re.search(r", s\[\d+:\d+\]$", l) for l in r)]
    assert runs and max(len(r) for r in runs) >= 16, f"staging loads are not batched: {[len(r) for r in runs]}"


def test_register_worker_operand_loads_are_batched(asm):
    # the register worker's staging: eight loads per thread in one batch
    runs = [r for r in _load_runs(_kernel(asm, "t")[0]) if all(re.search(r", s\[\d+:\d+\]$", l) for l in r)]
    assert any(len(r) == 8 for r in runs), [len(r) for r in runs]


def _vregs(op):
    m = re.match(r"v\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", op)
    return {int(m.group(1))} if m else set()


@pytest.mark.parametrize("tmpl", ["t", "f"])
def test_wide_store_data_not_overwritten_next(asm, tmpl):
    # a vector store of more than 8 bytes reads its data registers a cycle
    # after it issues: the next instruction must not write them
    body = [l for l in _kernel(asm, tmpl)[0] if l and not l.startswith((";", "."))]
    bad = []
    for i, l in enumerate(body[:-1]):
        if l.startswith(("global_store_dwordx3", "global_store_dwordx4", "buffer_store_dwordx4")):
            data = _vregs(l.split(None, 1)[1].split(",")[1].strip())
            nxt = body[i + 1]
            if nxt.startswith("v_") and not nxt.startswith(("v_readlane", "v_cmp")):
                dst = nxt.split(None, 1)[1].split(",")[0].strip()
                if _vregs(dst) & data:
                    bad.append((l, nxt))
    assert not bad, bad[:5]


def _sregs(op):
    m = re.match(r"s\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", op)
    return {int(m.group(1))} if m else set()


@pytest.mark.parametrize("tmpl", ["t", "f"])
def test_asm_memory_base_not_written_by_valu_just_before(asm, tmpl):
    # a vector instruction writing a scalar register needs five wait states
    # before a memory instruction reads it as an address; the compiler's hazard
    # check does not see into inline asm, so the asm must provide them
    body = [l for l in _kernel(asm, tmpl)[0] if l and not l.startswith(".") and not l.endswith(":")]
    inside, bad, checked = False, [], 0
    for i, l in enumerate(body):
        if l.startswith(";;#ASMSTART"):
            inside = True
            continue
        if l.startswith(";;#ASMEND"):
            inside = False
            continue
        if not inside or not l.startswith(("global_", "buffer_")):
            continue
        ops = [o.strip() for o in l.split(None, 1)[1].split(",")]
        sbase = set().union(*[_sregs(o) for o in ops[2:3]]) if len(ops) > 2 else set()
        if not sbase:
            continue
        checked += 1
        waits, j = 0, i - 1
        while j >= 0 and waits < 5:
            prev = body[j]
            j -= 1
            if prev.startswith(";"):
                continue
            if prev.startswith("s_nop"):
                waits += int(prev.split()[1]) + 1
                continue
            if prev.startswith("v_"):
                dsts = [o.strip() for o in prev.split(None, 1)[1].split(",")[:2]]
                if any(_sregs(d) & sbase for d in dsts):
                    bad.append((prev, l))
                    break
            waits += 1
    assert checked, "no asm memory instruction with a scalar base found"
    assert not bad, bad[:5]


# ---- the dense-product and chain-head kernels

CSRC = os.path.join(ROOT, "conditional_draft_tree_dominotree_amd", "csrc")


def _compile(src, tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("codegen") / (os.path.basename(src) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", "-o", str(out), os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _body(asm_text, prefix):
    lines = asm_text.split("\n")
    label = re.compile(re.escape(prefix) + r"\w*:")
    starts = [i for i, l in enumerate(lines) if label.match(l)]
    assert starts, prefix
    out = []
    for s in starts:
        name = lines[s].split(":")[0]
        end = next(i for i in range(s, len(lines)) if "s_endpgm" in lines[i])
        meta = re.search(re.escape(name) + r"\.private_seg_size, (\d+)", asm_text)
        out.append((name, [l.strip() for l in lines[s:end]], int(meta.group(1)) if meta else None))
    return out


@pytest.mark.parametrize("src,prefix", [("gemm.hip", "_ZN2dt20gemm_bf16_big_kernel"),
                                        ("gemm.hip", "_ZN2dt19gemm_lm_half_kernel"),
                                        ("gemm.hip", "_ZN2dt19gemm_lm_topk_kernel"),
                                        ("gemm.hip", "_ZN2dt16lm_select_kernel"),
                                        ("chain.hip", "_ZN2dt25chain_correct_mfma_kernel"),
                                        ("chain.hip", "_ZN2dt20chain_correct_kernel")])
def test_dense_kernels_use_no_scratch(tmp_path_factory, src, prefix):
    # a spill in these kernels costs a memory round trip per loop iteration
    for name, body, priv in _body(_compile(src, tmp_path_factory), prefix):
        assert not any(l.startswith("scratch_") for l in body), name
        if priv is not None:
            assert priv == 0, name


@pytest.mark.parametrize("prefix,vm", [("_ZN2dt20gemm_bf16_big_kernel", 16), ("_ZN2dt19gemm_lm_half_kernel", 6),
                                       ("_ZN2dt19gemm_lm_topk_kernel", 6)])
def test_gemm_waits_for_its_oldest_stage_only(tmp_path_factory, prefix, vm):
    # the main loop waits for its oldest stage of operand loads only (the
    # later stages stay in flight: two of 8 loads, one of 6), then the barrier
    for name, body, _ in _body(_compile("gemm.hip", tmp_path_factory), prefix):
        assert any(l.startswith(f"s_waitcnt vmcnt({vm})") for l in body), name
        assert sum(l.startswith("global_load_lds_dwordx4") for l in body) >= 2 * vm, name
