"""TEST INFRASTRUCTURE ONLY — fp64 CPU oracle for chunked-prefill causal attention.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and this package imports nothing from the GPU library.

What is computed follows the VPP technical review (English edition), §2.2
Eq. (1) (scaled dot-product attention), the causal rule stated beside it in
§2.2, and §2.3 (a chunk at offset ``past_len`` attends to the cache of every
earlier chunk plus itself).  The arithmetic lives in ``attn_oracle.c`` (plain
C, IEEE fp64, two passes); this module only marshals numpy arrays.

Inputs are numpy arrays of float32, float64 (used for values that fp32 cannot
hold exactly, such as dequantized fp8), or uint16 holding bfloat16 bit
patterns (widened exactly to fp64 inside the C code).  Layouts are logical:
``q [chunk_len, Hq, d]``, ``k [kv_len, Hkv, d]``, ``v [kv_len, Hkv, dv]``.

Every function here is pinned by the CPU tests (closed forms, invariants,
brute force on tiny inputs, a library routine on the special case with no
past, and hand-derived golden values); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
# CHUNKATTN_ORACLE_LIB selects another build (the host-sanitized one); it is then used as it is.
_LIB_PATH = os.environ.get("CHUNKATTN_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2


def build(path: str | None = None, extra=(), cc: str = "gcc") -> str:
    """Compile attn_oracle.c (-O3, OpenMP, no fast-math, no FMA contraction); ``extra`` flags and another
    compiler serve the host-sanitized build."""
    path = path or _LIB_PATH
    tmp = path + ".tmp"
    cmd = [cc, "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", *extra, _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, path)
    return path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.environ.get("CHUNKATTN_ORACLE_LIB") and (
            not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.orc_attend_rows.restype = ctypes.c_int
    lib.orc_attend_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_int64,
        ctypes.c_int64, i64p, i32p, ctypes.c_int64, ctypes.c_int64,
        f64p, f64p, ctypes.c_int32]
    lib.orc_merge.restype = ctypes.c_int
    lib.orc_merge.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                              f64p, f64p, f64p, f64p]
    _lib = lib
    return lib


def _dtype_code(*arrays) -> int:
    kinds = {a.dtype for a in arrays}
    if kinds == {np.dtype(np.float32)}:
        return F32
    if kinds == {np.dtype(np.uint16)}:
        return BF16
    if kinds == {np.dtype(np.float64)}:
        return F64
    raise TypeError(f"oracle inputs must all be float32, all float64 or all uint16 (bf16 bits), got {kinds}")


def attend_rows(q, k, v, past_len: int, scale: float, tok, head,
                key_range=None, threads: int | None = None):
    """Attention output and LSE for the query rows ``(tok[r], head[r])``.

    Row r is query token ``tok[r]`` of the chunk (absolute position
    ``past_len + tok[r]``) and query head ``head[r]``; it attends to keys
    ``0 .. past_len + tok[r]`` of the logical cache, intersected with
    ``key_range = (lo, hi)`` when given.  Returns ``out [n_rows, dv]`` and
    ``lse [n_rows]`` (natural log) in fp64.
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dt = _dtype_code(q, k, v)
    c, hq, d = q.shape
    kv_len, hkv, d2 = k.shape
    assert d2 == d and v.shape[:2] == (kv_len, hkv)
    dv = v.shape[2]
    tok = np.ascontiguousarray(tok, dtype=np.int64)
    head = np.ascontiguousarray(head, dtype=np.int32)
    n = tok.shape[0]
    assert head.shape == (n,)
    out = np.empty((n, dv), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    lo, hi = (-1, -1) if key_range is None else key_range
    rc = _load().orc_attend_rows(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, dt, c, kv_len, hq, hkv, d, dv,
        float(scale), int(past_len), n,
        tok.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        head.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        int(lo), int(hi),
        out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        lse.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        int(threads or 0))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (row out of range or key beyond kv_len)")
    return out, lse


def chunk_attention(q, k, v, past_len: int, scale: float, key_range=None,
                    threads: int | None = None):
    """Every row of one chunk: ``out [chunk_len, Hq, dv]``, ``lse [Hq, chunk_len]``."""
    c, hq, _ = q.shape
    tok = np.repeat(np.arange(c, dtype=np.int64), hq)
    head = np.tile(np.arange(hq, dtype=np.int32), c)
    out, lse = attend_rows(q, k, v, past_len, scale, tok, head, key_range, threads)
    return out.reshape(c, hq, -1), lse.reshape(c, hq).T.copy()


def merge(o_parts, lse_parts):
    """LSE merge of partials over disjoint key ranges.

    ``o_parts [S, n_rows, dv]`` and ``lse_parts [S, n_rows]`` (fp64) →
    ``out [n_rows, dv]``, ``lse [n_rows]``.
    """
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    s, n, dv = o_parts.shape
    assert lse_parts.shape == (s, n)
    out = np.empty((n, dv), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    f64p = ctypes.POINTER(ctypes.c_double)
    rc = _load().orc_merge(s, n, dv, o_parts.ctypes.data_as(f64p), lse_parts.ctypes.data_as(f64p),
                           out.ctypes.data_as(f64p), lse.ctypes.data_as(f64p))
    if rc != 0:
        raise ValueError("oracle merge rejected its arguments")
    return out, lse


def bf16_bits_to_f64(bits):
    """Exact widening of bf16 bit patterns (uint16) to fp64, for comparisons."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
