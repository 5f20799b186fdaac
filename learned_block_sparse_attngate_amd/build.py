"""Build libseer.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python -m learned_block_sparse_attngate_amd.build [--verbose]
The library lands next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_NAME = "libseer.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["attn_kernels.hip", "gate_kernels.hip", "decode_kernels.hip", "seer_api.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep fp32 arithmetic on unpacked VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the gfx950 library)")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every HIP source for gfx950 and link libseer.so; returns its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="seer_build_") as tmp:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            # hipcc's host pass does not know the gfx feature above; that warning is harmless
            lines = [ln for ln in out.splitlines() if "not a recognized feature for this target" not in ln]
            if lines and (verbose or p.returncode != 0):
                print("\n".join(lines), file=sys.stderr)
            if p.returncode != 0:
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed on {failed}")
        tmp_lib = os.path.join(tmp, LIB_NAME)
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        shutil.move(tmp_lib, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
