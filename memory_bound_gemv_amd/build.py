"""Compile the HIP library libmbg.so for gfx950 in-tree with hipcc."""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmbg.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed FP32 instructions stay off: plain float code only.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]
# step.hip is built once per compiled model family (-DMBG_STEP_SHAPE=i), in parallel
STEP_SHAPES = 4
SOURCES = [("step.hip", i) for i in range(STEP_SHAPES)] + [("ops.hip", None), ("api.cpp", None)]


def source_digest() -> str:
    """SHA-256 over the library's sources, the public header and the flags:
    names the kernel build that a stored counter measurement belongs to."""
    h = hashlib.sha256()
    names = sorted(os.listdir(CSRC))
    for n in names:
        if n.endswith((".hip", ".cpp", ".h")):
            h.update(n.encode())
            with open(os.path.join(CSRC, n), "rb") as f:
                h.update(f.read())
    with open(os.path.join(INCLUDE, "mbg.h"), "rb") as f:
        h.update(f.read())
    h.update(" ".join(f for f in FLAGS if f not in (INCLUDE, CSRC)).encode())
    return h.hexdigest()[:16]


def _compile(item, extra) -> str:
    src, shape = item
    tag = "" if shape is None else f".shape{shape}"
    obj = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    defs = [] if shape is None else [f"-DMBG_STEP_SHAPE={shape}"]
    cmd = [HIPCC, *FLAGS, *defs, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra_flags=(), verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)
