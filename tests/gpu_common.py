"""Helpers for the GPU parity tests: seeded inputs, paged pools, comparisons.

The expected values always come from the fp64 CPU oracle fed with the very
same input tensors the GPU reads (copied to the host).  Paged pools are
filled through the library's cache-write kernel, whose layout is itself
checked bitwise against a torch restatement of the pool layout.
"""
from __future__ import annotations

import math
import sys
import time

import numpy as np
import torch

import oracle
from chunked_prefill_causal_amd import _lib as L
from chunked_prefill_causal_amd import inputs

BF16_TOL = 1.5e-2      # max abs error, bf16 inputs with fp32 accumulation
F32_TOL = 1e-4         # max abs error, fp32 inputs
LSE_TOL = 1e-3         # natural-log LSE, fp32 on the GPU


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def require_gpu() -> None:
    assert torch.cuda.is_available(), "GPU test started without a visible GPU"
    L.lib()   # raises when the HIP library is missing


def torch_dtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


def seq_kv(n_tokens, kv_heads, d, dv, dtype, seed):
    """Host logical K [n, Hkv, d] and V [n, Hkv, dv] for one sequence."""
    return inputs.normal((n_tokens, kv_heads, d), seed, dtype), inputs.normal((n_tokens, kv_heads, dv), seed + 1, dtype)


class Pool:
    """A paged pool holding one or more sequences, filled by the cache-write kernel."""

    def __init__(self, num_blocks, kv_heads, d, dv, dtype, poison=True):
        self.k, self.v = L.paged_pool(num_blocks, kv_heads, d, dv, dtype)
        if poison:   # unowned blocks and block tails hold NaN; no output may see them
            self.k.fill_(float("nan"))
            self.v.fill_(float("nan"))
        self.num_blocks = num_blocks

    def append(self, k_host, v_host, table, start=0):
        L.chunkattn_kv_append(k_host.cuda(), v_host.cuda(), start, table, self.k, self.v)


def single_seq_pool(k_host, v_host, seed, poison=True):
    n = k_host.shape[0]
    needed = max(1, math.ceil(n / L.BLOCK_SIZE))
    table = torch.from_numpy(inputs.block_table(needed, seed)).cuda()
    pool = Pool(inputs.pool_size(needed), k_host.shape[1], k_host.shape[2], v_host.shape[2], k_host.dtype, poison)
    pool.append(k_host, v_host, table)
    return pool, table


def max_err(gpu, ref) -> float:
    g = gpu.detach().float().cpu().numpy().astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - r))) if g.size else 0.0


def oracle_chunk(q_host, k_host, v_host, past, scale, threads=None):
    return oracle.chunk_attention(inputs.to_oracle(q_host), inputs.to_oracle(k_host), inputs.to_oracle(v_host),
                                  past, scale, threads=threads)


def oracle_rows(q_host, k_host, v_host, past, scale, tok, head, threads=None):
    return oracle.attend_rows(inputs.to_oracle(q_host), inputs.to_oracle(k_host), inputs.to_oracle(v_host),
                              past, scale, tok, head, threads=threads)


def build_batch(q_lens, kv_lens, hq, hkv, d, dv, seed, poison=True):
    """Per-sequence seeded K/V and queries placed in one pool with disjoint random blocks."""
    n = len(q_lens)
    max_blocks = max(math.ceil(k / 64) for k in kv_lens)
    needed = [math.ceil(k / 64) for k in kv_lens]
    total = sum(needed)
    pool_blocks = inputs.pool_size(total)
    perm = inputs.block_table(total, seed, pool_blocks)
    pool = Pool(pool_blocks, hkv, d, dv, torch.bfloat16, poison=poison)
    tables = np.zeros((n, max_blocks), dtype=np.int32)
    seqs = []
    off = 0
    for s in range(n):
        tables[s, : needed[s]] = perm[off: off + needed[s]]
        off += needed[s]
        k, v = seq_kv(kv_lens[s], hkv, d, dv, "bf16", seed + 10 * s + 1)
        q = inputs.normal((q_lens[s], hq, d), seed + 10 * s + 5, "bf16")
        seqs.append((q, k, v))
    tables_d = torch.from_numpy(tables).cuda()
    for s in range(n):
        pool.append(seqs[s][1], seqs[s][2], tables_d[s])
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q_all = torch.cat([x[0] for x in seqs]) if cu[-1] else torch.empty((0, hq, d), dtype=torch.bfloat16)
    return pool, tables_d, cu, q_all, seqs
