"""Build libapb.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m sparse_block_attention_amd.build

Each source compiles to its own object under _build/ (in parallel), then one
link produces sparse_block_attention_amd/libapb.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libapb.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # No packed fp32 instructions (v_pk_*_f32) in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-source compiler options.  The attention kernel is scheduled with LLVM's
# max-ILP strategy and without the post-register-allocation scheduler, which
# otherwise reorders the interleaving of MFMAs with loads and softmax work that the
# kernel's scheduling hints ask for.  At the Llama-3.1-8B host shape, in interleaved
# rounds of 20 launches, this is 0.9% faster than max-ILP alone, which is 0.3-0.5%
# faster than the default strategy; iterative-ILP and max-memory-clause were 2-4%
# slower, and clustering or the exact interleaving solver changed no instruction.
EXTRA_FLAGS = {
    "block_attention.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp",
                            "-mllvm", "-enable-post-misched=0"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, hipcc: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *HIP_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-I", INCLUDE, "-I", CSRC, "-c", src,
           "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc, "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libapb.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
