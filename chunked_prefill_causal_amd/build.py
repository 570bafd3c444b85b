"""Build libchunkattn.so for gfx950 with hipcc (in-tree, next to this file).

Every HIP source compiles to an object under ``_build/`` (in parallel), then
one hipcc link produces ``chunked_prefill_causal_amd/libchunkattn.so``.
Packed-FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libchunkattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["prefill.hip", "prefill_paged.hip", "decode.hip", "kv_append.hip", "mla.hip", "mla_prefill.hip", "api.cpp", "schedule.cpp", "alp.cpp"]
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # the direct-to-LDS loads set m0 in inline asm, which clang flags as a reserved register
         "-Wno-inline-asm",
         "-I", INCLUDE, "-I", CSRC]


# Per-source flags.  The MLA decode kernel keeps its matrix accumulators in
# ordinary VGPRs: it rescales them with vector ALU ops, and accumulator
# registers would be copied out and back on every loop iteration.
EXTRA = {"mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
