"""Build libsegattn.so for gfx950 in-tree with hipcc.

Usage: python -m attention_segmented_kv_amd.build [--verbose] [--debug | --all]
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
SOURCES = ["api.hip", "prefill.hip", "decode.hip", "append.hip", "linear.hip", "allocator.cpp"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32 on its own.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(ROOT, "include")]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


# Variants: "release" (libsegattn.so) and "debug" (libsegattn_debug.so: SEG_ATTN_DEBUG, whose
# entry points check the segment tables on the host before every attention launch).
VARIANTS = {
    "release": ("libsegattn.so", []),
    "debug": ("libsegattn_debug.so", ["-DSEG_ATTN_DEBUG=1", "-g"]),
}


def library_file(variant: str = "release") -> str:
    return os.path.join(PKG, VARIANTS[variant][0])


def build(verbose: bool = False, extra_flags=(), variant: str = "release") -> str:
    """Compile every HIP source for gfx950 and link the variant's library next to this file."""
    name, vflags = VARIANTS[variant]
    bdir = os.path.join(BUILD, variant)
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *HIP_FLAGS, *vflags, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    lib = os.path.join(PKG, name)
    tmp = lib + ".tmp"
    _run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


def build_all(verbose: bool = False):
    """Both variants."""
    return [build(verbose, variant=v) for v in VARIANTS]


if __name__ == "__main__":
    if "--all" in sys.argv:
        print("\n".join(build_all(verbose="--verbose" in sys.argv)))
    else:
        print(build(verbose="--verbose" in sys.argv, variant="debug" if "--debug" in sys.argv else "release"))
