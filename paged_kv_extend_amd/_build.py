"""Build libpkv.so (HIP for gfx950) in-tree with hipcc."""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")
# the debug build: the same kernels, with the C ABI checking every index array
# on the device before use (PKV_ERR_RANGE) -- one host sync per call
LIB_DEBUG = os.path.join(PKG, "libpkv_debug.so")
SOURCES = ["api.cpp", "index_build.hip", "kv_cache.hip", "plan.hip", "attention.hip", "attention_dl.hip",
           "decode.hip", "debug_check.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         # no packed fp32 instructions from the compiler
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# per-source additions to FLAGS (none at present)
SOURCE_FLAGS = {}


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    tag = "_debug" if debug else ""
    out = os.path.join(OBJ, os.path.splitext(src)[0] + tag + ".o")
    cmd = ["hipcc", *FLAGS, *SOURCE_FLAGS.get(src, []), *(["-DPKV_DEBUG"] if debug else []), "-c",
           os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if verbose:
        print(" ".join(cmd))
    return out


def _link(objs, lib: str) -> None:
    tmp = lib + f".tmp{os.getpid()}"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every HIP source and link libpkv.so and libpkv_debug.so (the C ABI
    built with PKV_DEBUG, the same kernels); returns the path of libpkv.so."""
    os.makedirs(OBJ, exist_ok=True)
    jobs_list = [(s, False) for s in SOURCES] + [("api.cpp", True)]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs_list))
    release = objs[:len(SOURCES)]
    _link(release, LIB)
    debug_api = objs[len(SOURCES)]
    _link([debug_api if o.endswith("api.o") else o for o in release], LIB_DEBUG)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
