"""Build libikbo.so (HIP C++ for gfx950) in-tree with hipcc.

    python -m broadcast_gemm_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libikbo.so")
SOURCES = ["ikbo_api.cpp", "lce_kernels.hip", "lce_fused.hip", "lce_rows.hip", "lce_stream.hip", "lce_noalloc.hip", "lce_backward.hip", "ikbo_fa.cpp",
           "fa_kernels.hip"]
ARCH = os.environ.get("IKBO_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source and link libikbo.so (always rebuilds)."""
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
              "-I", CSRC, "-Wall", "-Wno-unused-function",
              # Packed fp32 VALU forms stay off in generated code.
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        cmd = [hipcc()] + common + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    objs = []
    for src, obj, proc in jobs:
        _, err = proc.communicate()
        msgs = "\n".join(l for l in (err or "").splitlines() if "packed-fp32-ops" not in l)
        if proc.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
