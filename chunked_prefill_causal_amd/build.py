"""Build libchunkattn.so for gfx950 with hipcc (in-tree, next to this file).

Every HIP source compiles to an object under ``_build/`` (in parallel), then
one hipcc link produces ``chunked_prefill_causal_amd/libchunkattn.so``.
Packed-FP32 instructions are disabled for all device code.

The two prefill kernels write m0 (the LDS destination of a direct-to-LDS load)
in one inline-asm statement and issue the load in a later one, with MFMAs in
between as the wait state the GFX9 m0 hazard needs.  That is sound only while
no code the compiler emits writes m0, so their device assembly is generated
beside the objects and checked before the link (``check_m0``).

``python chunked_prefill_causal_amd/build.py --sanitize`` builds a host-side
ASan + UBSan copy of the library and of the CPU oracle under ``_build/san``
and runs the CPU test suite against them.
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

# Sources whose loads read an m0 written by an earlier asm statement.
M0_SPLIT = ["prefill_paged.hip", "mla_prefill.hip"]


# Host-only AddressSanitizer + UndefinedBehaviorSanitizer build (device code is built as usual).  It
# links against clang's shared sanitizer runtime, which the process must preload (see `sanitizer_env`).
SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -shared-libsan "
             "-Xarch_host -fno-omit-frame-pointer -Xarch_host -g").split()
# the CPU oracle is plain C built by clang, so these need no -Xarch_host
ORACLE_SAN_FLAGS = ("-fsanitize=address,undefined -fno-sanitize-recover=undefined -shared-libsan "
                    "-fno-omit-frame-pointer -g").split()
LLVM = os.environ.get("ROCM_LLVM", "/opt/rocm/lib/llvm")


def _compile(src: str, sanitize: bool = False) -> str:
    out_dir = SAN_DIR if sanitize else BUILD_DIR
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *(SAN_FLAGS if sanitize else []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _device_asm(src: str) -> str:
    """The gfx950 assembly of one source, as the object build compiles it."""
    out = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "--cuda-device-only", "-S", "-x", "hip", os.path.join(CSRC, src),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stderr}")
    with open(out) as f:
        return f.read()


def check_m0(asm: str, name: str) -> int:
    """Check the two rules the split direct-to-LDS loads rely on, over every function of ``asm``: each write
    of m0 comes from an inline-asm statement of ours (so none lands between our m0 write and the load that
    reads it), and each direct-to-LDS load has at least one instruction between it and the last m0 write
    (the wait state of the GFX9 hazard).  Returns the number of loads checked; raises on a violation."""
    in_asm = False
    since_m0 = None                                  # instructions since the last m0 write
    loads = 0
    for lineno, raw in enumerate(asm.splitlines(), 1):
        line = raw.split(";")[0].strip() if not raw.lstrip().startswith(";;#ASM") else raw.strip()
        if line.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if line.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not line or line.startswith(".") or line.endswith(":"):
            if line.endswith(":") and not line.startswith("."):
                since_m0 = None                      # a label: the path into it is not this one
            continue
        op, _, rest = line.partition(" ")
        dst = rest.split(",")[0].strip()
        if dst == "m0" and not op.startswith(("global_", "buffer_", "ds_")):
            if not in_asm:
                raise RuntimeError(f"{name}:{lineno}: the compiler writes m0 ({line}); the split direct-to-LDS "
                                   "loads would read the wrong LDS destination")
            since_m0 = 0
            continue
        if op.startswith("global_load_lds"):
            if since_m0 == 0:
                raise RuntimeError(f"{name}:{lineno}: direct-to-LDS load right after an m0 write")
            loads += 1
        if since_m0 is not None:
            since_m0 += 1
    return loads


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build libchunkattn.so in place; with ``sanitize`` a host-sanitized copy under _build/san instead."""
    out_dir = SAN_DIR if sanitize else BUILD_DIR
    os.makedirs(out_dir, exist_ok=True)
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES) + len(M0_SPLIT)) as ex:
        asm_jobs = [(src, ex.submit(_device_asm, src)) for src in M0_SPLIT]
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
        for src, job in asm_jobs:
            check_m0(job.result(), src)
    lib = os.path.join(SAN_DIR, "libchunkattn.so") if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(SAN_FLAGS if sanitize else []), "-o", tmp, *objs]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def sanitizer_env() -> dict:
    """Environment that runs Python with the sanitized library and oracle: clang's shared ASan runtime
    preloaded (the interpreter is not instrumented), leak checks off (the interpreter's own allocations),
    and the library / oracle paths pointed at the _build/san copies."""
    import glob
    rt = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not rt:
        raise RuntimeError(f"no clang ASan runtime under {LLVM}")
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt[-1]
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:detect_odr_violation=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["LD_LIBRARY_PATH"] = os.path.join(LLVM, "lib") + ":" + env.get("LD_LIBRARY_PATH", "")
    env["CHUNKATTN_LIB"] = os.path.join(SAN_DIR, "libchunkattn.so")
    env["CHUNKATTN_ORACLE_LIB"] = os.path.join(SAN_DIR, "liboracle.so")
    return env


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--sanitize", action="store_true",
                    help="host ASan + UBSan build of the library and the CPU oracle under _build/san, then run "
                         "the CPU test suite with them")
    args = ap.parse_args()
    if not args.sanitize:
        build(verbose=True)
    else:
        build(verbose=True, sanitize=True)
        sys.path.insert(0, ROOT)
        import oracle
        oracle.build(os.path.join(SAN_DIR, "liboracle.so"), extra=ORACLE_SAN_FLAGS, cc=os.path.join(LLVM, "bin", "clang"))
        r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu",
                            "-p", "no:cacheprovider"], env=sanitizer_env(), cwd=ROOT)
        sys.exit(r.returncode)
