"""Build libattn.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m exact_attention_14_amd.build [--define NAME=VALUE ...] [--out PATH]

Sources are compiled in parallel into ``_build/`` at the repository root and
linked into ``exact_attention_14_amd/libattn.so``.  Every call recompiles.
``--define`` passes build parameters to every compile (the forward's tile
shape: ATTN_FWD_BLOCK_K, ATTN_FWD_WAVES_NONE, ATTN_FWD_WAVES_MASKED; see
csrc/plan.hpp) and ``--out`` writes such a variant elsewhere, e.g.
``exact_attention_14_amd/variants/libattn_bc128.so``, which the binding loads
when the environment variable EXACT_ATTN_LIB names it (tile-shape sweeps).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")

ARCH = "gfx950"
HIP_SOURCES = ["fwd_kernel.hip", "bwd_kernels.hip", "decode_kernel.hip", "launch.hip"]
# The backward's key-major kernel keeps its dV/dK accumulators in AGPRs
# (inline-asm matrix instructions) and its score tiles in VGPRs; the
# compiler's own matrix instructions must then use the VGPR form, or it would
# place the score tiles in AGPRs and copy them out for the vector code.
EXTRA_FLAGS = {"bwd_kernels.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
CXX_SOURCES = ["validate.cpp"]

# Packed fp32 arithmetic is disabled for every device compile.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}", f"-I{CSRC}"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose: bool = False, defines=(), out: str = LIB) -> str:
    tag = "".join(f"_{d}" for d in defines).replace("=", "")
    build_dir = os.path.join(BUILD, "variant" + tag) if defines else BUILD
    os.makedirs(build_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    hipcc = _hipcc()
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        objs.append(obj)
        jobs.append([hipcc, *HIP_FLAGS, *dflags, *EXTRA_FLAGS.get(src, []), "-c",
                     os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        objs.append(obj)
        jobs.append(["g++", *CXX_FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for text in ex.map(_run, jobs):
            if verbose and text.strip():
                print(text)
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    tmp = out + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


def _main(argv) -> None:
    import argparse
    ap = argparse.ArgumentParser(description="build libattn.so for gfx950")
    ap.add_argument("-v", action="store_true", help="print compiler output")
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE",
                    help="build parameter passed to every compile")
    ap.add_argument("--out", default=LIB, help="library path to write")
    a = ap.parse_args(argv)
    for d in a.define:
        if not d.startswith("ATTN_") or "=" not in d:
            raise SystemExit(f"--define takes ATTN_NAME=VALUE, got {d!r}")
    print(build(verbose=a.v, defines=a.define, out=a.out))


if __name__ == "__main__":
    _main(sys.argv[1:])
