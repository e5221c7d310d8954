"""Build libkda.so in-tree with hipcc for gfx950.

Each translation unit is compiled to an object in ``_build/`` (in parallel),
then linked into ``gated_delta_rule_90_amd/libkda.so``.  Every call rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkda.so")

# (source, object name, extra flags): the recurrent kernel is built once per key
# dimension so that its instantiations compile in parallel
SOURCES = [("kda_api.cpp", "kda_api", []), ("kda_noalloc.cpp", "kda_noalloc", []), ("kda_decode.hip", "kda_decode", []),
           ("kda_chunked.hip", "kda_chunked", []), ("kda_chunked_f32.hip", "kda_chunked_f32", []),
           ("kda_backward.hip", "kda_backward", []), ("kda_gated.hip", "kda_gated", [])] + \
    [("kda_recurrent.hip", f"kda_recurrent_dk{dk}", [f"-DKDA_RECURRENT_DK={dk}"]) for dk in (16, 32, 64, 128)]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def _compile(entry) -> str:
    src, name, extra = entry
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
