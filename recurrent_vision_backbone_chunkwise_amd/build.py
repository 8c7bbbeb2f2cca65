"""Builds libgtr_gla.so (the HIP kernels and the C ABI) in-tree for gfx950.

Run ``python -m recurrent_vision_backbone_chunkwise_amd.build`` or call
``build()``.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgtr_gla.so")

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
SOURCES = ["gla_kernels.hip", "gla_api.cpp", "gla_bwd.cpp", "gla_profile.cpp", "swiglu.hip"]


def code_tokens(text: str) -> str:
    """C/C++ source without its comments, with every run of whitespace as one space (string and
    character literals kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c.isspace():
            j = i
            while j < n and text[j].isspace():
                j += 1
            out.append(" ")
            i = j
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest() -> str:
    """Short digest of the kernel and host sources: ties measurements to the code they measured.
    Comments and layout do not count, so editing them leaves measurements attached."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                h.update(name.encode())
                h.update(code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(hipcc: str, src: str, extra_flags: list[str], verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC,
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{msg}")
    if verbose:
        print(" ".join(cmd), flush=True)
        if msg.strip():
            print(msg, flush=True)
    return obj


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    # the sources compile independently, so in parallel (each is one hipcc process)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda src: _compile(hipcc, src, extra_flags or [], verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-lrocblas", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
