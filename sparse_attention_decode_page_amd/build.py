"""Compile libspdec.so (all HIP kernels and the C ABI) for gfx950, in-tree,
and libspdec_probe.so (the gather-read ceiling probe that bench.py times next
to the kernels; not part of the library's ABI).

Each source compiles to its own object in parallel (`_build/` beside this
file), then one link step per library makes the shared libraries.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libspdec.so")
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libspdec_probe.so")
PROBE_SOURCES = ["probe.hip"]
SOURCES = ["abi.hip", "grid.hip", "meta.hip", "select.hip", "decode.hip", "path.hip", "slice.hip", "verify.hip", "shared.hip", "speculative.hip",
           "acceptance.hip", "control.hip", "check.hip", "noalloc.hip", "monitor.hip"]

# Packed-FP32 VALU instructions are switched off for all device code.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libspdec")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd[-3:])}")
    if verbose and res.stderr.strip():
        lines = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = list(SOURCES) + list(PROBE_SOURCES)
    objs = [os.path.join(OBJ_DIR, s.replace(".hip", ".o")) for s in srcs]
    cc = hipcc()
    cmds = [[cc, *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), max(1, min(os.cpu_count() or 1, 16)))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for path, names in ((LIB_PATH, SOURCES), (PROBE_LIB_PATH, PROBE_SOURCES)):
        tmp = path + ".tmp"
        lib_objs = [os.path.join(OBJ_DIR, s.replace(".hip", ".o")) for s in names]
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *lib_objs, "-o", tmp], verbose)
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
