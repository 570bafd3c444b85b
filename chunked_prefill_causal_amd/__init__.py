"""Chunked-prefill causal attention for MI355X (gfx950).

The compute path is ``libchunkattn.so`` (hand-written HIP kernels behind the C
ABI in ``include/chunkattn.h``); this package binds it with the same names.
Importing the package does not load the library; the first call does, and
raises if the library has not been built.
"""
from ._lib import (  # noqa: F401
    BLOCK_SIZE,
    ChunkAttnError,
    chunk_attn_varlen,
    chunk_prefill_attn,
    chunkattn_kv_append,
    chunkattn_prefill_auto_splits,
    chunkattn_prefill_workspace_size,
    chunkattn_varlen_workspace_size,
    lib,
    paged_pool,
    version,
)
