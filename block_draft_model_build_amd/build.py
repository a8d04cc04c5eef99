"""Builds libdflash.so in-tree with hipcc for gfx950 (cross-compiles without a GPU).

    python block_draft_model_build_amd/build.py      # or build() from Python
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdflash.so")
SOURCES = ["dflash.hip", "plan.hip", "profile.hip", "verify.hip", "attn_bwd.hip", "ctx_bwd.hip", "body_bwd.hip", "lm_bwd.hip", "optim.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdflash)")


def compile_flags():
    return ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source and link libdflash.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(OBJ, exist_ok=True)

    def one(src):
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        cmd = [hipcc, *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = (r.stdout + r.stderr).strip()
        # hipcc's host pass does not know the packed-fp32 feature name; that note is harmless.
        noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
        out = "\n".join(x for x in out.splitlines() if noise not in x)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{out}")
        if out and verbose:
            print(out, file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
