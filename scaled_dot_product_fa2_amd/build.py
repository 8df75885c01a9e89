"""Build the gfx950 attention library in-tree: ``scaled_dot_product_fa2_amd/libsdpa_fa2.so``.

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions disabled, then linked
into one shared library exporting the C ABI of ``include/sdpa_fa2.h``.  Run as
``python -m scaled_dot_product_fa2_amd.build`` (or through ``__graft_entry__.build()``).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libsdpa_fa2.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["fwd_bf16.hip", "fwd_f32.hip", "decode.hip", "bwd_bf16.hip", "api.cpp"]
ARCH = "gfx950"
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
    # no packed fp32 (v_pk_*_f32) code generation anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build)")


def _compile(src: str, resource_report: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if resource_report and src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    out = "\n".join(ln for ln in out.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, resource_report: bool = False) -> str:
    """Compile every source and link the library; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        logs = list(ex.map(lambda s: _compile(s, resource_report), SOURCES))
    if verbose:
        for s, log in zip(SOURCES, logs):
            if log:
                print(f"--- {s}\n{log}")
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose=True, resource_report="--resources" in sys.argv)
    print(path)
