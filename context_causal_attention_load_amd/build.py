"""Builds libcpattn.so in-tree with hipcc for gfx950.

Usage: ``python -m context_causal_attention_load_amd.build`` (or ``__graft_entry__.build()``).
Objects go to ``_build/`` at the repository root; the library lands next to this file.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libcpattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "permute.hip", "attn_fwd.hip", "decode.hip", "decode_int8.hip", "attn_bwd.hip"]

# Packed fp32 VALU ops are disabled for all device code; the compiler would otherwise form them
# from ordinary float code.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcpattn.so)")


def _compile(hipcc, src, obj, extra):
    cmd = [hipcc, *HIP_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False, extra_flags=()):
    """Compile every HIP source and link libcpattn.so (always rebuilds)."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o")
            jobs.append(ex.submit(_compile, hipcc, src, obj, list(extra_flags)))
        objs = [j.result() for j in jobs]
    tmp = OUT + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
