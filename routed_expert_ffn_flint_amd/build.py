"""Builds libflint_moe.so (HIP kernels for gfx950 + the C ABI) in this directory.

    python -m routed_expert_ffn_flint_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libflint_moe.so")
SOURCES = ["route.hip", "expert.hip", "stream.hip", "stream_mx4.hip", "tiled.hip", "fused.hip", "abi.cpp",
           "static_ws.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the Flint MoE library needs ROCm's hipcc to build")


def build(verbose: bool = False, extra_flags=(), lib: str = LIB) -> str:
    """Compile every source for gfx950 and link the shared library at ``lib``
    (hipcc ``extra_flags`` added to every compile).  Always recompiles (the
    build is a few tens of seconds)."""
    out_dir = os.path.join(os.path.dirname(os.path.abspath(lib)), "_build")
    os.makedirs(out_dir, exist_ok=True)
    common = [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # keep the backend from forming packed fp32 instructions by itself
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", f"-I{os.path.join(HERE, '..', 'include')}",
    ] + list(extra_flags)
    def compile_one(src):
        obj = os.path.join(out_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc()] + common + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        return obj

    # the sources compile independently: in parallel, a few at a time
    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = f"{lib}.tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
