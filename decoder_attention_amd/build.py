"""Build the HIP library libgemma_attn.so in-tree (gfx950).

    python -m decoder_attention_amd.build          # compile every source, link

Two builds of the same sources, both written next to this file:
  libgemma_attn.so         the library;
  libgemma_attn_ldsnan.so  the debug build (GA_LDS_POISON=1): every kernel
                           fills its LDS with NaN bytes before use, so a read
                           of LDS it never wrote shows in the outputs.
Objects go to decoder_attention_amd/_build/ (the debug build's to
_build/ldsnan/).  Every call recompiles.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgemma_attn.so")
LIB_LDSNAN = os.path.join(PKG, "libgemma_attn_ldsnan.so")

HIP_SOURCES = ["prologue.hip", "prefill.hip", "decode.hip", "gemma_attn_api.hip"]
CXX_SOURCES = ["host_logic.cpp"]
ARCH = "gfx950"


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _flags() -> list[str]:
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # packed fp32 arithmetic stays off for every kernel of this library
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def build(jobs: int | None = None) -> str:
    """Compile both builds (the library and its LDS-poisoning debug build) and
    link them; returns the library's path."""
    hipcc = _hipcc()
    dbg_dir = os.path.join(BUILD, "ldsnan")
    os.makedirs(dbg_dir, exist_ok=True)
    cmds, objs, dbg_objs = [], [], []
    for src in HIP_SOURCES + CXX_SOURCES:
        stem = os.path.splitext(src)[0]
        obj = os.path.join(BUILD, stem + ".o")
        objs.append(obj)
        lang = [] if src.endswith(".hip") else ["-x", "c++"]
        cmds.append([hipcc, *_flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        if src.endswith(".hip"):
            dobj = os.path.join(dbg_dir, stem + ".o")
            dbg_objs.append(dobj)
            cmds.append([hipcc, *_flags(), "-DGA_LDS_POISON=1", "-c", os.path.join(CSRC, src), "-o", dobj])
        else:
            dbg_objs.append(obj)   # host code has no LDS
    # the longest compiles (decode.hip) first
    cmds.sort(key=lambda c: "decode.hip" not in " ".join(c))
    with ThreadPoolExecutor(jobs or min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(_run, cmds))
    for target, parts in ((LIB, objs), (LIB_LDSNAN, dbg_objs)):
        tmp = target + ".tmp"
        _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *parts, "-o", tmp])
        os.replace(tmp, target)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=None)
    a = ap.parse_args()
    print(build(a.j))


if __name__ == "__main__":
    if shutil.which(_hipcc()) is None and not os.path.exists(_hipcc()):
        sys.exit("hipcc not found")
    main()
