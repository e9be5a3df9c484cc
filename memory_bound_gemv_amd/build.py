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


def _code_tokens(text: str) -> str:
    """C/C++ source with every run of whitespace and comments turned into
    one separator (a newline if the run holds one outside a comment, else a
    space), string and character literals kept as written: what the
    compiler sees, so that a comment or layout edit does not rename the
    build."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif c.isspace() or text.startswith("//", i) or text.startswith("/*", i):
            newline = False
            while i < n:
                if text[i].isspace():
                    newline = newline or text[i] == "\n"
                    i += 1
                elif text.startswith("//", i):
                    j = text.find("\n", i)
                    i = n if j < 0 else j
                elif text.startswith("/*", i):
                    j = text.find("*/", i + 2)
                    i = n if j < 0 else j + 2
                else:
                    break
            out.append("\n" if newline else " ")
        else:
            out.append(c)
            i += 1
    return "".join(out).strip()


def source_digest() -> str:
    """SHA-256 over the library's sources (comments and layout aside), the
    public header and the flags: names the kernel build that a stored
    counter measurement belongs to."""
    h = hashlib.sha256()
    names = sorted(os.listdir(CSRC))
    for n in names:
        if n.endswith((".hip", ".cpp", ".h")):
            h.update(n.encode())
            with open(os.path.join(CSRC, n), encoding="utf-8") as f:
                h.update(_code_tokens(f.read()).encode())
    with open(os.path.join(INCLUDE, "mbg.h"), encoding="utf-8") as f:
        h.update(_code_tokens(f.read()).encode())
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
