"""Build libxattn.so for gfx950 with hipcc (in-tree, next to this file).

Usage: python block_sparse_attention_xattn_amd/build.py [--verbose]
(run by path: the package import would load the library being rebuilt)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libxattn.so")
# peak-rate microbenchmarks (measurement only), a library of their own
PEAKS_LIB = os.path.join(HERE, "libxattn_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "score.hip", "select.hip", "attn.hip", "dusa1.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay disabled on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# the debug build: the same sources with the kernels' bounds checks counted
# (-DXATTN_DEBUG=1, include/xattn_debug.h), a library of its own
DEBUG_LIB = os.path.join(HERE, "libxattn_debug.so")
DEBUG_BUILD = os.path.join(BUILD, "debug")


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    obj = os.path.join(DEBUG_BUILD if debug else BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *(["-DXATTN_DEBUG=1"] if debug else []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(DEBUG_BUILD, exist_ok=True)
    jobs = [(s, False) for s in SOURCES + PEAKS_SOURCES] + [(s, True) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = dict(zip(jobs, ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs)))
    _link([objs[(s, False)] for s in SOURCES], LIB)
    _link([objs[(s, False)] for s in PEAKS_SOURCES], PEAKS_LIB)
    _link([objs[(s, True)] for s in SOURCES], DEBUG_LIB)
    return LIB


def build_asan_check() -> str:
    """The host-ASan check of the C ABI's validation layer: api.hip's host code
    and tests/native/abi_check.cpp built with AddressSanitizer (host code only;
    the device code of every object is unchanged), linked with the library's
    other objects into an executable that needs no GPU. Returns its path."""
    out_dir = os.path.join(BUILD, "asan")
    os.makedirs(out_dir, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        build()
    asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    api_o = os.path.join(out_dir, "api.o")
    chk_o = os.path.join(out_dir, "abi_check.o")
    exe = os.path.join(out_dir, "xattn_abi_check")
    steps = [
        [HIPCC, *FLAGS, *asan, "-c", os.path.join(CSRC, "api.hip"), "-o", api_o],
        [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", *asan, "-x", "c++", "-c",
         os.path.join(ROOT, "tests", "native", "abi_check.cpp"), "-o", chk_o],
        [HIPCC, "--offload-arch=gfx950", *asan, chk_o, api_o, *objs, "-o", exe],
    ]
    for cmd in steps:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("ASan check build failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return exe


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
    if "--asan-check" in sys.argv:
        print(build_asan_check())
