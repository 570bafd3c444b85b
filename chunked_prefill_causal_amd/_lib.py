"""ctypes binding of libchunkattn: argument marshalling only.

Every step of the attention path runs in the HIP kernels behind
``include/chunkattn.h``.  This module turns torch tensors into device
pointers, allocates outputs and workspaces with torch (plumbing), passes the
current HIP stream, and raises :class:`ChunkAttnError` on a non-OK status.
There is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CHUNKATTN_LIB selects another build of the library (e.g. the host-sanitized one).
LIB_PATH = os.environ.get("CHUNKATTN_LIB") or os.path.join(_HERE, "libchunkattn.so")

CA_OK, CA_EINVAL, CA_EUNSUPPORTED, CA_ERANGE, CA_EWORKSPACE, CA_EHIP = 0, -1, -2, -3, -4, -5
CA_F32, CA_BF16 = 0, 1
CA_KV_CONTIGUOUS, CA_KV_PAGED = 0, 1
CA_SCHED_CPP, CA_SCHED_VPP, CA_SCHED_VPP_ASYNC = 0, 1, 2
CA_MLA_BF16, CA_MLA_FP8 = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20     # CHUNKATTN_NOALLOC_SCRATCH_BYTES
BLOCK_SIZE = 64
MLA_LATENT, MLA_ROPE = 512, 64

EXPORTED = ("ca_prefill_opts_init", "chunk_prefill_attn", "chunkattn_prefill_workspace_size",
            "chunkattn_prefill_contiguous_workspace_size",
            "chunkattn_prefill_auto_splits", "chunk_attn_varlen", "chunk_attn_varlen_noalloc",
            "chunkattn_varlen_workspace_size",
            "chunkattn_kv_append", "chunkattn_sched_simulate", "chunkattn_sched_drain_pack",
            "chunkattn_alp_features", "chunkattn_alp_init", "chunkattn_alp_predict", "chunkattn_alp_update",
            "chunkattn_mla_block_bytes", "chunkattn_mla_decode_workspace_size", "chunkattn_mla_kv_append",
            "chunk_mla_decode", "chunkattn_mla_prefill_workspace_size", "chunk_mla_prefill",
            "chunkattn_last_error", "chunkattn_version")


class ChunkAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libchunkattn status {status}: {message}")
        self.status = status


class PrefillOpts(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("out_dtype", ctypes.c_int), ("head_dim_v", ctypes.c_int32),
                ("kv_layout", ctypes.c_int), ("kv_capacity", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("block_table_len", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("lse_out", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("num_splits", ctypes.c_int32), ("k_stride_tok", ctypes.c_int64),
                ("k_stride_head", ctypes.c_int64), ("v_stride_tok", ctypes.c_int64),
                ("v_stride_head", ctypes.c_int64)]


ALP_FEATURES = 5


class AlpState(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_double * ALP_FEATURES), ("info", ctypes.c_double * (ALP_FEATURES * ALP_FEATURES)),
                ("rhs", ctypes.c_double * ALP_FEATURES), ("lambda_", ctypes.c_double), ("n_obs", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    L.ca_prefill_opts_init.argtypes = [ctypes.POINTER(PrefillOpts)]
    L.ca_prefill_opts_init.restype = None
    L.chunk_prefill_attn.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, f32, vp, ctypes.POINTER(PrefillOpts), vp]
    L.chunk_prefill_attn.restype = ctypes.c_int
    L.chunkattn_prefill_workspace_size.argtypes = [i64, i32, i32, i32]
    L.chunkattn_prefill_workspace_size.restype = sz
    L.chunkattn_prefill_contiguous_workspace_size.argtypes = [i64, i64, i32, i32, i32, i32, ctypes.c_int, i32]
    L.chunkattn_prefill_contiguous_workspace_size.restype = sz
    L.chunkattn_prefill_auto_splits.argtypes = [i64, i64, i32, i32]
    L.chunkattn_prefill_auto_splits.restype = i32
    L.chunk_attn_varlen.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, i32,
                                    vp, vp, sz, vp]
    L.chunk_attn_varlen.restype = ctypes.c_int
    L.chunk_attn_varlen_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp,
                                            i32, vp, vp]
    L.chunk_attn_varlen_noalloc.restype = ctypes.c_int
    L.chunkattn_varlen_workspace_size.argtypes = [vp, vp, i32, i32, i32, i32]
    L.chunkattn_varlen_workspace_size.restype = sz
    L.chunkattn_kv_append.argtypes = [vp, vp, i64, i64, i32, i32, i32, ctypes.c_int, vp, i32, i32, vp, vp,
                                      ctypes.POINTER(ctypes.c_int64), vp]
    L.chunkattn_kv_append.restype = ctypes.c_int
    f64 = ctypes.c_double
    L.chunkattn_sched_simulate.argtypes = [i32, i32, vp, vp, f64, i32, vp, vp, vp, vp]
    L.chunkattn_sched_simulate.restype = ctypes.c_int
    L.chunkattn_sched_drain_pack.argtypes = [i32, f64, i32, vp, vp]
    L.chunkattn_sched_drain_pack.restype = i32
    L.chunkattn_alp_features.argtypes = [i32, vp, vp, i32, i32, vp]
    L.chunkattn_alp_features.restype = ctypes.c_int
    L.chunkattn_alp_init.argtypes = [ctypes.POINTER(AlpState), f64, f64]
    L.chunkattn_alp_init.restype = ctypes.c_int
    L.chunkattn_alp_predict.argtypes = [ctypes.POINTER(AlpState), vp]
    L.chunkattn_alp_predict.restype = f64
    L.chunkattn_alp_update.argtypes = [ctypes.POINTER(AlpState), vp, f64, vp]
    L.chunkattn_alp_update.restype = ctypes.c_int
    L.chunkattn_mla_block_bytes.argtypes = [i32]
    L.chunkattn_mla_block_bytes.restype = sz
    L.chunkattn_mla_decode_workspace_size.argtypes = [vp, i32, i32, i32]
    L.chunkattn_mla_decode_workspace_size.restype = sz
    L.chunkattn_mla_kv_append.argtypes = [vp, vp, i64, i64, i32, vp, i32, i32, vp, vp]
    L.chunkattn_mla_kv_append.restype = ctypes.c_int
    L.chunk_mla_decode.argtypes = [vp, vp, i32, vp, i32, i32, vp, vp, i32, i32, f32, vp, i32, vp, vp, sz, vp]
    L.chunk_mla_decode.restype = ctypes.c_int
    L.chunkattn_mla_prefill_workspace_size.argtypes = [i64, i64, i32]
    L.chunkattn_mla_prefill_workspace_size.restype = sz
    L.chunk_mla_prefill.argtypes = [vp, vp, i32, vp, i32, i32, i64, i64, i32, f32, vp, i32, vp, vp, sz, vp]
    L.chunk_mla_prefill.restype = ctypes.c_int
    L.chunkattn_last_error.argtypes = []
    L.chunkattn_last_error.restype = ctypes.c_char_p
    L.chunkattn_version.argtypes = []
    L.chunkattn_version.restype = i32
    _lib = L
    return L


def _check(status: int) -> None:
    if status != CA_OK:
        raise ChunkAttnError(status, lib().chunkattn_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


# The C calls take bare pointers and sizes, so they cannot see a tensor's
# shape, dtype or strides; these checks refuse, before the library is called,
# a tensor laid out other than the call assumes (the kernels would read or
# write outside it).
def _expect(t, name: str, shape=None, dtype=None, dense: bool = True) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(a) for a in allowed)}")
    if dense and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _expect_on_gpu(**tensors) -> None:
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


def _expect_paged_pool(k_pool, v_pool, kv_heads: int, head_dim: int, head_dim_v: int, dtype) -> None:
    """The pools :func:`paged_pool` makes: K ``[nb, kv_heads, d/x, 64, x]``, V ``[nb, kv_heads, 64/x, dv, x]``
    with x values per 16 bytes."""
    x = elems_per_16b(dtype)
    nb = k_pool.shape[0]
    _expect(k_pool, "k_pool", (nb, kv_heads, head_dim // x, BLOCK_SIZE, x), dtype)
    _expect(v_pool, "v_pool", (nb, kv_heads, BLOCK_SIZE // x, head_dim_v, x), dtype)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return CA_BF16
    if dt == torch.float32:
        return CA_F32
    raise TypeError(f"unsupported dtype {dt}")


def elems_per_16b(dt: torch.dtype) -> int:
    return 16 // torch.empty((), dtype=dt).element_size()


def paged_pool(num_blocks: int, kv_heads: int, head_dim: int, head_dim_v: int, dtype, device="cuda"):
    """Allocate (uninitialised) K and V pools in the library's paged layout."""
    x = elems_per_16b(dtype)
    k = torch.empty((num_blocks, kv_heads, head_dim // x, BLOCK_SIZE, x), dtype=dtype, device=device)
    v = torch.empty((num_blocks, kv_heads, BLOCK_SIZE // x, head_dim_v, x), dtype=dtype, device=device)
    return k, v


def version() -> int:
    return lib().chunkattn_version()


def chunkattn_sched_simulate(kind: int, tau, comm: float = 0.0, request=None, pack: bool = True) -> dict:
    """Two-rank CPP / VPP / VPP-Async schedule of chunks with per-stage latencies ``tau`` (host only).

    Returns start and end times of every (chunk, virtual stage) as ``[n, 4]``
    float64 arrays, the busy time of each rank and the makespan.
    """
    import numpy as np

    t = np.ascontiguousarray(tau, dtype=np.float64)
    n = t.shape[0]
    req = None if request is None else np.ascontiguousarray(request, dtype=np.int32)
    start = np.empty((n, 4), dtype=np.float64)
    end = np.empty((n, 4), dtype=np.float64)
    busy = np.empty(2, dtype=np.float64)
    span = ctypes.c_double()
    _check(lib().chunkattn_sched_simulate(kind, n, t.ctypes.data if n else None,
                                          None if req is None else req.ctypes.data, float(comm), int(bool(pack)),
                                          start.ctypes.data, end.ctypes.data, busy.ctypes.data, ctypes.byref(span)))
    return {"start": start, "end": end, "busy": busy, "makespan": span.value}


def chunkattn_alp_features(q_lens, kv_lens, heads: int, kv_heads: int):
    """ALP feature vector of a batch (FastPP notes §2.3): [1, sum Lpast*Lpre/1e6, sum Lpre^2/1e6, sum Ldec/1e3]
    and the prefill launch's fill term for ``heads`` / ``kv_heads``."""
    import numpy as np

    q = np.ascontiguousarray(q_lens, dtype=np.int32)
    kv = np.ascontiguousarray(kv_lens, dtype=np.int32)
    x = np.empty(ALP_FEATURES, dtype=np.float64)
    _check(lib().chunkattn_alp_features(q.shape[0], q.ctypes.data if q.shape[0] else None,
                                        kv.ctypes.data if kv.shape[0] else None, int(heads), int(kv_heads),
                                        x.ctypes.data))
    return x


class AlpPredictor:
    """Recursive least-squares fit of the ALP coefficients (information form), state in the library's struct."""

    def __init__(self, lam: float = 1.0, delta: float = 1e6):
        self.state = AlpState()
        _check(lib().chunkattn_alp_init(ctypes.byref(self.state), float(lam), float(delta)))

    def predict(self, x) -> float:
        import numpy as np

        xv = np.ascontiguousarray(x, dtype=np.float64)
        return lib().chunkattn_alp_predict(ctypes.byref(self.state), xv.ctypes.data)

    def update(self, x, measured: float) -> float:
        import numpy as np

        xv = np.ascontiguousarray(x, dtype=np.float64)
        err = ctypes.c_double()
        _check(lib().chunkattn_alp_update(ctypes.byref(self.state), xv.ctypes.data, float(measured), ctypes.byref(err)))
        return err.value

    @property
    def theta(self):
        return list(self.state.theta)


def chunkattn_sched_drain_pack(n_chunks: int, t: float, tau_next) -> tuple[int, float]:
    """Alg. 2: leading chunks of the next request that fit in the (N + 1) t drain window, and what is left."""
    import numpy as np

    tn = np.ascontiguousarray(tau_next, dtype=np.float64)
    left = ctypes.c_double()
    j = lib().chunkattn_sched_drain_pack(n_chunks, float(t), tn.shape[0], tn.ctypes.data if tn.shape[0] else None,
                                         ctypes.byref(left))
    if j < 0:
        _check(j)
    return j, left.value


def chunkattn_prefill_workspace_size(chunk_len: int, heads: int, head_dim_v: int, num_splits: int) -> int:
    return lib().chunkattn_prefill_workspace_size(chunk_len, heads, head_dim_v, num_splits)


def chunkattn_prefill_contiguous_workspace_size(past_len: int, chunk_len: int, heads: int, kv_heads: int,
                                                head_dim: int, head_dim_v: int, num_splits: int,
                                                dtype: int = CA_BF16) -> int:
    return lib().chunkattn_prefill_contiguous_workspace_size(past_len, chunk_len, heads, kv_heads, head_dim,
                                                             head_dim_v, dtype, num_splits)


def chunkattn_prefill_auto_splits(past_len: int, chunk_len: int, heads: int, kv_heads: int) -> int:
    return lib().chunkattn_prefill_auto_splits(past_len, chunk_len, heads, kv_heads)


def chunk_prefill_attn(q, k_cache, v_cache, past_len: int, scale: float | None = None, *,
                       kv_layout: str = "contiguous", block_table=None, num_blocks: int | None = None,
                       kv_heads: int | None = None, head_dim_v: int | None = None, out=None, out_dtype=None,
                       return_lse: bool = False, lse=None, num_splits: int = 0, workspace=None,
                       kv_capacity: int | None = None, relayout: bool = True, stream=None):
    """One chunk of causal prefill attention; see ``chunk_prefill_attn`` in the header.

    ``q`` is ``[chunk_len, heads, head_dim]``.  Contiguous caches are
    ``[capacity, kv_heads, head_dim(_v)]``; paged pools come from
    :func:`paged_pool` with ``block_table`` an int32 device tensor.  A
    contiguous cache may be a strided view (e.g. K and V sliced out of a
    fused QKV tensor) as long as its last dim is dense.  For a
    bf16 contiguous cache the workspace allocated here has room for the
    library to re-lay the prefix for the paged kernel (``relayout=False``
    sizes it for split partials only, so the cache is read in place).
    Returns ``out`` (and ``lse [heads, chunk_len]`` when requested).
    """
    if q.dim() != 3:
        raise ValueError(f"q: expected [chunk_len, heads, head_dim], got shape {tuple(q.shape)}")
    _expect(q, "q", dtype=(torch.bfloat16, torch.float32))
    c, heads, d = q.shape
    paged = kv_layout == "paged"
    if paged:
        nb, hkv = k_cache.shape[0], k_cache.shape[1]
        dv = v_cache.shape[3]
        _expect_paged_pool(k_cache, v_cache, hkv, d, dv, q.dtype)
        _expect(block_table, "block_table", dtype=torch.int32)
    else:
        if k_cache.dim() != 3 or v_cache.dim() != 3:
            raise ValueError("contiguous caches are [capacity, kv_heads, head_dim(_v)]")
        hkv, dv = k_cache.shape[1], v_cache.shape[2]
        nb = 0
        if k_cache.shape[2] != d or v_cache.shape[1] != hkv:
            raise ValueError("k_cache / v_cache disagree with q's head_dim or with each other's kv_heads")
        _expect(k_cache, "k_cache", dtype=q.dtype, dense=False)
        _expect(v_cache, "v_cache", dtype=q.dtype, dense=False)
    if kv_heads is not None and kv_heads != hkv:
        raise ValueError("kv_heads disagrees with the cache shape")
    if head_dim_v is not None and head_dim_v != dv:
        raise ValueError("head_dim_v disagrees with the value cache shape")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((c, heads, dv), dtype=out_dtype, device=q.device)
    _expect(out, "out", (c, heads, dv), (torch.bfloat16, torch.float32))
    if return_lse and lse is None:
        lse = torch.empty((heads, c), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, "lse", (heads, c), torch.float32)
    if workspace is None and not paged and relayout and c > 0:
        need = chunkattn_prefill_contiguous_workspace_size(past_len, c, heads, hkv, d, dv, num_splits,
                                                           _dtype_code(q.dtype))
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if num_splits == 0 and workspace is None:
        auto = chunkattn_prefill_auto_splits(past_len, c, heads, hkv)
        if auto > 1:
            workspace = torch.empty(chunkattn_prefill_workspace_size(c, heads, dv, auto),
                                    dtype=torch.uint8, device=q.device)
    elif num_splits > 1 and workspace is None:
        workspace = torch.empty(max(1, chunkattn_prefill_workspace_size(c, heads, dv, num_splits)),
                                dtype=torch.uint8, device=q.device)
    o = PrefillOpts()
    lib().ca_prefill_opts_init(ctypes.byref(o))
    o.dtype = _dtype_code(q.dtype)
    o.out_dtype = _dtype_code(out.dtype)
    o.head_dim_v = dv
    o.kv_layout = CA_KV_PAGED if paged else CA_KV_CONTIGUOUS
    if paged:
        o.block_table = _ptr(block_table)
        o.block_table_len = block_table.numel()
        o.num_blocks = nb if num_blocks is None else num_blocks
    else:
        o.kv_capacity = k_cache.shape[0] if kv_capacity is None else kv_capacity
        for t, name in ((k_cache, "k"), (v_cache, "v")):
            if t.stride(2) != 1:
                raise ValueError(f"{name}_cache: the head dim must be dense")
            if not t.is_contiguous():
                setattr(o, f"{name}_stride_tok", _stride(t, 0))
                setattr(o, f"{name}_stride_head", _stride(t, 1))
    o.lse_out = _ptr(lse)
    if workspace is not None:
        o.workspace = _ptr(workspace)
        o.workspace_bytes = _nbytes(workspace)
    o.num_splits = num_splits
    _expect_on_gpu(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table if paged else None, out=out,
                   lse=lse, workspace=workspace)
    _check(lib().chunk_prefill_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), past_len, c, heads, hkv, d,
                                    float(scale), _ptr(out), ctypes.byref(o), _stream(stream)))
    return (out, lse) if return_lse else out


def _stride(t, dim: int) -> int:
    """Element stride of a [tokens, heads, d] view along `dim`; torch may report any stride for a size-1
    dimension, which is never stepped, so that case gets the dense value.  A broadcast (stride-0)
    dimension is refused here: the ABI reads a zero stride as "dense", which would step past the
    tensor's storage."""
    if t.shape[dim] > 1:
        if t.stride(dim) <= 0:
            raise ValueError(f"a cache view broadcast along dim {dim} (stride {t.stride(dim)}) is not supported")
        return t.stride(dim)
    return t.shape[2] * (t.shape[1] if dim == 0 else 1)


def _host_i32(x):
    t = torch.as_tensor(x, dtype=torch.int32).cpu().contiguous()
    return t


def chunkattn_varlen_workspace_size(cu_seqlens_q, kv_lens, heads: int, kv_heads: int, head_dim_v: int) -> int:
    cu, kv = _host_i32(cu_seqlens_q), _host_i32(kv_lens)
    return lib().chunkattn_varlen_workspace_size(cu.data_ptr(), kv.data_ptr(), kv.numel(), heads, kv_heads,
                                                 head_dim_v)


def chunk_attn_varlen(q, k_pool, v_pool, block_tables, cu_seqlens_q, kv_lens, scale: float | None = None, *,
                      num_blocks: int | None = None, out=None, out_dtype=None, return_lse: bool = False, lse=None,
                      workspace=None, cu_seqlens_q_dev=None, kv_lens_dev=None, stream=None):
    """Mixed prefill + decode batch over a paged pool; see ``chunk_attn_varlen``.

    ``cu_seqlens_q`` and ``kv_lens`` are host sequences (int32); device copies
    are made unless given.  ``block_tables`` is ``[num_seqs, max_blocks]`` int32
    on the device.  The output is bf16 or fp32 (``out_dtype``, or that of ``out``).
    """
    if q.dim() != 3:
        raise ValueError(f"q: expected [total_q, heads, head_dim], got shape {tuple(q.shape)}")
    _expect(q, "q", dtype=torch.bfloat16)
    total_q, heads, d = q.shape
    hkv, dv = k_pool.shape[1], v_pool.shape[3]
    _expect_paged_pool(k_pool, v_pool, hkv, d, dv, q.dtype)
    cu, kv = _host_i32(cu_seqlens_q), _host_i32(kv_lens)
    if cu.numel() != kv.numel() + 1:
        raise ValueError("cu_seqlens_q needs one more entry than kv_lens")
    _expect(block_tables, "block_tables", (kv.numel(), block_tables.shape[-1]), torch.int32)
    n = kv.numel()
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if cu_seqlens_q_dev is None:
        cu_seqlens_q_dev = cu.to(q.device)
    if kv_lens_dev is None:
        kv_lens_dev = kv.to(q.device)
    _expect(cu_seqlens_q_dev, "cu_seqlens_q_dev", (n + 1,), torch.int32)
    _expect(kv_lens_dev, "kv_lens_dev", (n,), torch.int32)
    if out is None:
        out = torch.empty((total_q, heads, dv), dtype=out_dtype or q.dtype, device=q.device)
    _expect(out, "out", (total_q, heads, dv), (torch.bfloat16, torch.float32))
    if return_lse and lse is None:
        lse = torch.empty((heads, total_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, "lse", (heads, total_q), torch.float32)
    if workspace is None:
        need = lib().chunkattn_varlen_workspace_size(cu.data_ptr(), kv.data_ptr(), n, heads, hkv, dv)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _expect_on_gpu(q=q, k_pool=k_pool, v_pool=v_pool, block_tables=block_tables, cu_seqlens_q_dev=cu_seqlens_q_dev,
                   kv_lens_dev=kv_lens_dev, out=out, lse=lse, workspace=workspace)
    _check(lib().chunk_attn_varlen(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
        k_pool.shape[0] if num_blocks is None else num_blocks, _ptr(cu_seqlens_q_dev), _ptr(kv_lens_dev),
        cu.data_ptr(), kv.data_ptr(), n, heads, hkv, d, dv, float(scale), _ptr(out), _dtype_code(out.dtype),
        _ptr(lse), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return (out, lse) if return_lse else out


def chunk_attn_varlen_noalloc(q, k_pool, v_pool, block_tables, cu_seqlens_q, kv_lens, scale: float | None = None, *,
                              out, cu_seqlens_q_dev, kv_lens_dev, num_blocks: int | None = None, lse=None,
                              stream=None):
    """``chunk_attn_varlen`` on the library's static per-device scratch (no workspace).

    For callers that cannot allocate: every tensor, the output and the device
    copies of the lengths included, must be passed in; this function creates
    none.  ``cu_seqlens_q`` and ``kv_lens`` are host sequences (int32); the
    output dtype (bf16 or fp32) is that of ``out``.
    """
    if q.dim() != 3:
        raise ValueError(f"q: expected [total_q, heads, head_dim], got shape {tuple(q.shape)}")
    _expect(q, "q", dtype=torch.bfloat16)
    total_q, heads, d = q.shape
    hkv, dv = k_pool.shape[1], v_pool.shape[3]
    _expect_paged_pool(k_pool, v_pool, hkv, d, dv, q.dtype)
    cu, kv = _host_i32(cu_seqlens_q), _host_i32(kv_lens)
    if cu.numel() != kv.numel() + 1:
        raise ValueError("cu_seqlens_q needs one more entry than kv_lens")
    _expect(block_tables, "block_tables", (kv.numel(), block_tables.shape[-1]), torch.int32)
    n = kv.numel()
    _expect(cu_seqlens_q_dev, "cu_seqlens_q_dev", (n + 1,), torch.int32)
    _expect(kv_lens_dev, "kv_lens_dev", (n,), torch.int32)
    _expect(out, "out", (total_q, heads, dv), (torch.bfloat16, torch.float32))
    if lse is not None:
        _expect(lse, "lse", (heads, total_q), torch.float32)
    _expect_on_gpu(q=q, k_pool=k_pool, v_pool=v_pool, block_tables=block_tables, cu_seqlens_q_dev=cu_seqlens_q_dev,
                   kv_lens_dev=kv_lens_dev, out=out, lse=lse)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().chunk_attn_varlen_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
        k_pool.shape[0] if num_blocks is None else num_blocks, _ptr(cu_seqlens_q_dev), _ptr(kv_lens_dev),
        cu.data_ptr(), kv.data_ptr(), kv.numel(), heads, hkv, d, dv, float(scale), _ptr(out), _dtype_code(out.dtype),
        _ptr(lse), _stream(stream)))
    return out


def chunkattn_kv_append(k_new, v_new, start_pos: int, block_table, k_pool, v_pool, *, num_blocks: int | None = None,
                        stream=None) -> None:
    """Write ``k_new [n, kv_heads, d]`` / ``v_new [n, kv_heads, dv]`` at positions start_pos..

    Either may be a strided view (e.g. sliced out of a fused QKV tensor) with a dense last dim."""
    if k_new.dim() != 3 or v_new.dim() != 3:
        raise ValueError("k_new / v_new are [n, kv_heads, head_dim(_v)]")
    n, hkv, d = k_new.shape
    dv = v_new.shape[2]
    if v_new.shape[:2] != (n, hkv):
        raise ValueError("k_new and v_new disagree on tokens or kv_heads")
    _expect(k_new, "k_new", dtype=(torch.bfloat16, torch.float32), dense=False)
    _expect(v_new, "v_new", dtype=k_new.dtype, dense=False)
    _expect_paged_pool(k_pool, v_pool, hkv, d, dv, k_new.dtype)
    _expect(block_table, "block_table", dtype=torch.int32)
    strides = None
    if not (k_new.is_contiguous() and v_new.is_contiguous()):
        if k_new.stride(2) != 1 or v_new.stride(2) != 1:
            raise ValueError("k_new / v_new: the head dim must be dense")
        strides = (ctypes.c_int64 * 4)(_stride(k_new, 0), _stride(k_new, 1), _stride(v_new, 0), _stride(v_new, 1))
    _expect_on_gpu(k_new=k_new, v_new=v_new, block_table=block_table, k_pool=k_pool, v_pool=v_pool)
    _check(lib().chunkattn_kv_append(_ptr(k_new), _ptr(v_new), start_pos, n, hkv, d, dv, _dtype_code(k_new.dtype),
                                     _ptr(block_table), block_table.numel(),
                                     k_pool.shape[0] if num_blocks is None else num_blocks,
                                     _ptr(k_pool), _ptr(v_pool), strides, _stream(stream)))


def chunkattn_mla_block_bytes(fmt: int) -> int:
    return lib().chunkattn_mla_block_bytes(fmt)


def mla_pool(num_blocks: int, fmt: int, device="cuda"):
    """Allocate (uninitialised) a paged MLA latent pool of ``num_blocks`` 64-token blocks, as bytes."""
    nbytes = chunkattn_mla_block_bytes(fmt)
    if nbytes == 0:
        raise ValueError(f"unknown MLA cache format {fmt}")
    return torch.empty((num_blocks, nbytes), dtype=torch.uint8, device=device)


def _expect_mla_pool(pool, fmt: int) -> None:
    nbytes = chunkattn_mla_block_bytes(fmt)
    if nbytes == 0:
        raise ValueError(f"unknown MLA cache format {fmt}")
    _expect(pool, "pool", (pool.shape[0], nbytes), torch.uint8)


def chunkattn_mla_kv_append(latent, rope, start_pos: int, block_table, pool, fmt: int, *,
                            num_blocks: int | None = None, stream=None) -> None:
    """Write ``latent [n, 512]`` / ``rope [n, 64]`` (bf16) at positions start_pos.. of one sequence."""
    n = latent.shape[0]
    _expect(latent, "latent", (n, MLA_LATENT), torch.bfloat16)
    _expect(rope, "rope", (n, MLA_ROPE), torch.bfloat16)
    _expect_mla_pool(pool, fmt)
    _expect(block_table, "block_table", dtype=torch.int32)
    _expect_on_gpu(latent=latent, rope=rope, block_table=block_table, pool=pool)
    _check(lib().chunkattn_mla_kv_append(_ptr(latent), _ptr(rope), start_pos, n, fmt, _ptr(block_table),
                                         block_table.numel(), pool.shape[0] if num_blocks is None else num_blocks,
                                         _ptr(pool), _stream(stream)))


def chunkattn_mla_decode_workspace_size(kv_lens, heads: int, fmt: int) -> int:
    kv = _host_i32(kv_lens)
    return lib().chunkattn_mla_decode_workspace_size(kv.data_ptr(), kv.numel(), heads, fmt)


def chunk_mla_decode(q, pool, fmt: int, block_tables, kv_lens, scale: float, *, num_blocks: int | None = None,
                     out=None, out_dtype=torch.bfloat16, return_lse: bool = False, lse=None, workspace=None,
                     kv_lens_dev=None, stream=None):
    """Absorbed MLA decode: ``q [num_seqs, heads, 576]`` bf16 against the latent pool; returns
    ``out [num_seqs, heads, 512]`` in ``out_dtype`` (bf16 or fp32; that of ``out`` when given) and
    ``lse [heads, num_seqs]`` fp32."""
    if q.dim() != 3:
        raise ValueError(f"q: expected [num_seqs, heads, {MLA_LATENT + MLA_ROPE}], got shape {tuple(q.shape)}")
    n, heads, _ = q.shape
    _expect(q, "q", (n, heads, MLA_LATENT + MLA_ROPE), torch.bfloat16)
    _expect_mla_pool(pool, fmt)
    kv = _host_i32(kv_lens)
    if kv.numel() != n:
        raise ValueError(f"kv_lens has {kv.numel()} entries for {n} sequences")
    _expect(block_tables, "block_tables", (n, block_tables.shape[-1]), torch.int32)
    if kv_lens_dev is None:
        kv_lens_dev = kv.to(q.device)
    _expect(kv_lens_dev, "kv_lens_dev", (n,), torch.int32)
    if out is None:
        out = torch.empty((n, heads, MLA_LATENT), dtype=out_dtype, device=q.device)
    _expect(out, "out", (n, heads, MLA_LATENT), (torch.bfloat16, torch.float32))
    if return_lse and lse is None:
        lse = torch.empty((heads, n), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, "lse", (heads, n), torch.float32)
    if workspace is None:
        need = lib().chunkattn_mla_decode_workspace_size(kv.data_ptr(), n, heads, fmt)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _expect_on_gpu(q=q, pool=pool, block_tables=block_tables, kv_lens_dev=kv_lens_dev, out=out, lse=lse,
                   workspace=workspace)
    _check(lib().chunk_mla_decode(
        _ptr(q), _ptr(pool), fmt, _ptr(block_tables), block_tables.shape[1],
        pool.shape[0] if num_blocks is None else num_blocks, _ptr(kv_lens_dev), kv.data_ptr(), n, heads,
        float(scale), _ptr(out), _dtype_code(out.dtype), _ptr(lse), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))
    return (out, lse) if return_lse else out


def chunkattn_mla_prefill_workspace_size(past_len: int, chunk_len: int, fmt: int) -> int:
    return lib().chunkattn_mla_prefill_workspace_size(int(past_len), int(chunk_len), fmt)


def chunk_mla_prefill(q, pool, fmt: int, block_table, past_len: int, scale: float, *,
                      num_blocks: int | None = None, out=None, out_dtype=torch.bfloat16, return_lse: bool = False,
                      lse=None, workspace=None, stream=None):
    """Absorbed MLA prefill of one chunk: ``q [chunk_len, heads, 576]`` bf16 for positions
    ``past_len ..`` of the sequence whose latent records the pool holds through ``block_table``;
    returns ``out [chunk_len, heads, 512]`` (``out_dtype``, or that of ``out``) and
    ``lse [heads, chunk_len]`` fp32.  An fp8 pool needs a workspace (allocated when not given)."""
    if q.dim() != 3:
        raise ValueError(f"q: expected [chunk_len, heads, {MLA_LATENT + MLA_ROPE}], got shape {tuple(q.shape)}")
    c, heads, _ = q.shape
    _expect(q, "q", (c, heads, MLA_LATENT + MLA_ROPE), torch.bfloat16)
    _expect_mla_pool(pool, fmt)
    _expect(block_table, "block_table", dtype=torch.int32)
    if out is None:
        out = torch.empty((c, heads, MLA_LATENT), dtype=out_dtype, device=q.device)
    _expect(out, "out", (c, heads, MLA_LATENT), (torch.bfloat16, torch.float32))
    if return_lse and lse is None:
        lse = torch.empty((heads, c), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, "lse", (heads, c), torch.float32)
    if workspace is None:
        need = chunkattn_mla_prefill_workspace_size(past_len, c, fmt)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    _expect_on_gpu(q=q, pool=pool, block_table=block_table, out=out, lse=lse, workspace=workspace)
    _check(lib().chunk_mla_prefill(
        _ptr(q), _ptr(pool), fmt, _ptr(block_table), block_table.shape[-1],
        pool.shape[0] if num_blocks is None else num_blocks, int(past_len), c, heads, float(scale), _ptr(out),
        _dtype_code(out.dtype), _ptr(lse), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return (out, lse) if return_lse else out
