"""Compile the HIP library in-tree: verify_router_gemv_amd/libmoe_round.so (gfx950).

    python -m verify_router_gemv_amd.build [--verbose]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_round.so")
SOURCES = (["moe_round.hip", "moe_validate.cpp"] + [f"moe_gemv_g{g}.hip" for g in (4, 8, 16, 32, 64)]
           + [f"moe_gemv_g{g}_s256.hip" for g in (4, 8, 16, 32, 64)])

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    "-munsafe-fp-atomics",                      # hardware fp32 atomic add for the scatter-add
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",   # no packed fp32 VALU ops
    "-fvisibility=hidden",
    "-Wall", "-Wno-unused-result",
]
# Per-source flags. moe_round.hip holds the prefill GEMMs, whose matrix-core results are folded
# into the accumulators on the vector ALUs: with the results in ordinary VGPRs (not accumulation
# registers) that costs no register-to-register copies. Its other matrix-core kernel (the fp64
# router GEMM) only stores its results.
SOURCE_FLAGS = {"moe_round.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "moe_gemv_g16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}  # the down tile's results fold on VALU


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), f"-I{INCLUDE}", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every translation unit in parallel, then link the shared library."""
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.time()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        for f in [pool.submit(_compile, s, o) for s, o in zip(SOURCES, objs)]:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"link failed ({res.returncode}): {' '.join(cmd)}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv or "-v" in sys.argv)
