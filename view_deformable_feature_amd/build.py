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
# read-bandwidth reference kernel for the benchmark (not part of the C ABI)
PROBE_PATH = os.path.join(PKG_DIR, "libbwprobe.so")
PROBE_SOURCE = os.path.join(PKG_DIR, "csrc", "bw_probe.hip")
SOURCES = [os.path.join(CSRC, f)
           for f in ("da_forward.hip", "da_backward.hip", "da_pack.hip", "da_api.cpp", "dcn.hip",
                     "dcn_api.cpp", "da_noalloc.hip")]
HEADERS = [os.path.join(INCLUDE, "deformagg.h"), os.path.join(INCLUDE, "dcn.h")] + [
    os.path.join(CSRC, f) for f in ("da_internal.h", "da_device.h", "da_pack.h", "dcn_internal.h",
                                    "host_errors.h")]
EXPORTS = os.path.join(CSRC, "exports.map")   # the C ABI is the only export
ARCH = "gfx950"


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        # no packed fp32 VALU instructions (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed: {' '.join(cmd[-3:])}")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libdeformagg.so; always recompiles."""
    from concurrent.futures import ThreadPoolExecutor
    hipcc = _hipcc()
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    objdir = os.path.join(PKG_DIR, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in SOURCES]
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run([hipcc, *compile_flags(), "-c", so[0], "-o", so[1]], verbose),
                    zip(SOURCES, objs)))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", *objs, "-o", tmp,
          f"-Wl,-rpath,{rocm_lib}", "-Wl,--no-undefined", f"-Wl,--version-script={EXPORTS}"],
         verbose)
    os.replace(tmp, LIB_PATH)
    tmp = PROBE_PATH + ".tmp"
    _run([hipcc, *compile_flags(), "-shared", PROBE_SOURCE, "-o", tmp, f"-Wl,-rpath,{rocm_lib}"],
         verbose)
    os.replace(tmp, PROBE_PATH)
    return LIB_PATH


def is_stale() -> bool:
    if not os.path.exists(LIB_PATH) or not os.path.exists(PROBE_PATH):
        return True
    if os.path.getmtime(PROBE_SOURCE) > os.path.getmtime(PROBE_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS + [EXPORTS])


if __name__ == "__main__":
    print(build(verbose=True))
