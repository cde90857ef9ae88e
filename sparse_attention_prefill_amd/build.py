"""Build libdsa.so (gfx950) in-tree with hipcc, and its checked twin libdsa_checked.so.

Usage: python -m sparse_attention_prefill_amd.build   (or call build_library() / build_all()).
Each .hip source compiles to an object in _build/ (_build/checked/ for the checked library),
then one shared library is linked next to this file. The checked library is the same sources
compiled with DSA_CHECKED: every gathered row id and data-dependent index is verified before
use and a failure is reported through err_flag (DSA_DEVERR_BOUNDS); it is for tests. Every call
compiles (there is no up-to-date check): the build is a few seconds per source on the CPU and
needs no GPU.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdsa.so")
LIB_CHECKED = os.path.join(HERE, "libdsa_checked.so")
SOURCES = ["api.hip", "metadata.hip", "rerange.hip", "indexer.hip", "topk.hip", "attention.hip", "probes.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed-fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src, checked=False):
    out_dir = os.path.join(BUILD, "checked") if checked else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + (["-DDSA_CHECKED"] if checked else []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    return obj


def build_library(verbose=False, checked=False):
    os.makedirs(os.path.join(BUILD, "checked") if checked else BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 7)) as ex:
        objs = list(ex.map(lambda src: _compile(src, checked), SOURCES))
    lib = LIB_CHECKED if checked else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


def build_all(verbose=False):
    """The product library, then the checked one."""
    build_library(verbose)
    return build_library(verbose, checked=True)


if __name__ == "__main__":
    build_all(verbose=True)
    sys.exit(0)
