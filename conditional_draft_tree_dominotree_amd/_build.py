"""Compile the HIP library libdominotree.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libdominotree.so")
OBJ = os.path.join(PKG, "_build")
SOURCES = ["api.hip", "topm.hip", "gemm.hip", "prepack.hip", "tree.hip", "verify.hip", "chain.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are not used anywhere in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(16, len(os.sched_getaffinity(0)))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


# host code under AddressSanitizer and UndefinedBehaviorSanitizer (the device
# code is built as usual, without them); the library then needs the clang ASan
# runtime preloaded into the process that loads it
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized(out_dir: str) -> str:
    """Compile every source with the host side sanitized (-O1 -g; the device
    side at -O3 as in the product build) into out_dir/libdominotree_san.so;
    returns its path."""
    os.makedirs(out_dir, exist_ok=True)
    flags = [*FLAGS, "-Xarch_host", "-O1", "-Xarch_host", "-g", *SANITIZE]

    def one(src: str) -> str:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    jobs = min(len(SOURCES), max(1, min(16, len(os.sched_getaffinity(0)))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    out = os.path.join(out_dir, "libdominotree_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return out


if __name__ == "__main__":
    build(verbose=True)
