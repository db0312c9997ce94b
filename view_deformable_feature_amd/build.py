"""Build libdeformagg.so in-tree for gfx950 with hipcc.

    python -m view_deformable_feature_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libdeformagg.so")
SOURCES = [os.path.join(CSRC, f) for f in ("da_forward.hip", "da_backward.hip", "da_api.cpp")]
HEADERS = [os.path.join(INCLUDE, "deformagg.h"), os.path.join(CSRC, "da_internal.h"),
           os.path.join(CSRC, "da_device.h")]
ARCH = "gfx950"


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # no packed fp32 VALU instructions (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source into libdeformagg.so (always recompiles)."""
    hipcc = _hipcc()
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, *compile_flags(), "-shared", *SOURCES, "-o", tmp,
           f"-Wl,-rpath,{rocm_lib}", "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {LIB_PATH}")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def is_stale() -> bool:
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
