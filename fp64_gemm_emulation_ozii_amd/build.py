"""Build the HIP library ``libozgemm.so`` for gfx950, in-tree.

Usage: ``python -m fp64_gemm_emulation_ozii_amd.build`` (or ``build()``).
Every call recompiles: each ``csrc/*.hip`` file becomes an object under
``_build/`` (compiled in parallel) and the objects are linked into
``fp64_gemm_emulation_ozii_amd/libozgemm.so``, replaced atomically.
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
OUT = os.path.join(PKG, "libozgemm.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["ozgemm.hip", "scale.hip", "residue.hip", "gemm_i8.hip", "crt.hip", "scheme1.hip", "accu.hip", "probe.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str, cc: str) -> str:
    cmd = [cc, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    # the host pass does not know the GPU target feature; that warning is expected
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    return "\n".join(noise)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        futs = {ex.submit(_compile, s, o, cc): s for s, o in zip(SOURCES, objs)}
        for fut in cf.as_completed(futs):
            warn = fut.result()
            if warn and verbose:
                print(f"[{futs[fut]}] {warn}", file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
