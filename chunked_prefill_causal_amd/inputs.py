"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws numbers and lays out bookkeeping arrays; it holds none of
the attention arithmetic.  Both the GPU path and the CPU oracle receive what
it produces, so it imports neither of them.

Workloads mirror the shapes the pages speak about: one long prompt split into
equal chunks that each attend to the cache of all earlier chunks (VPP
technical review, English edition, §2.3 and the 128K / 512K prefill runs of
its §3), grouped-query and MLA-shaped heads (its §5 model list), a paged KV
pool of 64-token blocks (GLM5.3 PP-split deployment notes, §1 and §7), and a
batch that mixes one prefill chunk with single-token decode requests
(Revisiting Pipeline Parallelism for LLM Serving, the preliminaries on chunks
and the three bubble kinds).

Recipe (fixed here, stated once):
  * values: iid N(0, 1) drawn as float32 with ``numpy.random.default_rng``;
    bf16 workloads round each draw to bfloat16 (round-to-nearest-even).
    Large tensors are filled in slabs of ``SLAB`` elements, each slab from its
    own child of ``SeedSequence(seed)``, so the values do not depend on the
    number of threads used.
  * device-side bulk draws (``normal_device``) use torch's seeded device
    generator; the oracle then reads the very same tensors copied to the host.
  * block table: a pool of ceil(1.25 * needed) blocks; the table is a seeded
    draw of ``needed`` distinct block ids.
  * decode context lengths: integers uniform on [lo, hi], both ends included.
  * MLA decode batch: per sequence, latents [kv, 512] then rotary parts
    [kv, 64] drawn N(0, 1) on the device from one seeded generator, rounded to
    bf16; queries [requests, heads, 576] N(0, 1) bf16 (GLM5.3 PP-split
    deployment notes §1, §4: one shared latent record per token).
  * MLA prefill prompt: latents [L, 512] then rotary parts [L, 64] of the one
    sequence from one seeded device generator (``mla_record_seed(w, 0)``),
    rounded to bf16; chunk k's queries [chunk, heads, 576] N(0, 1) bf16 from
    ``chunk_seeds(w, k)``.
  * sampled rows: every chunk's first and last token, tokens on both sides of
    every 64- and 128-token tile boundary (a bounded subset when there are
    many), and a seeded uniform fill; heads uniform.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

SLAB = 1 << 22
BLOCK_SIZE = 64


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    seq_len: int
    chunk_len: int
    heads: int
    kv_heads: int
    head_dim: int
    head_dim_v: int
    dtype: str                 # "f32" or "bf16"
    kv_layout: str             # "contiguous" or "paged"
    seed: int
    sample_rows: int = 0       # 0: compare every row
    # mixed prefill + decode batch
    decode_requests: int = 0
    decode_ctx: tuple = (0, 0)
    prefill_past: int = 0
    scale_dim: int = 0         # softmax scale 1/sqrt(scale_dim); 0: 1/sqrt(head_dim)

    @property
    def n_chunks(self) -> int:
        return math.ceil(self.seq_len / self.chunk_len) if self.chunk_len else 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.scale_dim or self.head_dim)


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", "L=2048 as 4 chunks of 512, 8 heads (MHA), d=64, fp32, contiguous KV",
        2048, 512, 8, 8, 64, 64, "f32", "contiguous", seed=101),
    "gqa_32k": Workload(
        "gqa_32k", "L=32768 as 8 chunks of 4096, 32 q heads / 8 KV heads, d=128, bf16, paged KV (64)",
        32768, 4096, 32, 8, 128, 128, "bf16", "paged", seed=202, sample_rows=4096),
    "gqa_128k": Workload(
        "gqa_128k", "L=131072 as 8 chunks of 16384, 64 q heads / 8 KV heads, d=128, bf16, paged KV (64)",
        131072, 16384, 64, 8, 128, 128, "bf16", "paged", seed=303, sample_rows=4096),
    "mla_512k": Workload(
        "mla_512k", "L=524288 as 16 chunks of 32768, 16 heads, d_qk=192 / d_v=128, bf16, paged KV (64)",
        524288, 32768, 16, 16, 192, 128, "bf16", "paged", seed=404, sample_rows=4096),
    "mixed": Workload(
        "mixed", "one 2048-token prefill chunk at past 65536 + 256 decodes, ctx ~ U[1024, 32768], "
        "32 q heads / 8 KV heads, d=128, bf16, paged KV (64)",
        65536 + 2048, 2048, 32, 8, 128, 128, "bf16", "paged", seed=505,
        decode_requests=256, decode_ctx=(1024, 32768), prefill_past=65536),
    # absorbed MLA decode: one 576-value record (512 latent + 64 rotary) per token shared by all
    # heads; the softmax scale is the expanded head's, 1/sqrt(128 + 64)
    "mla_decode": Workload(
        "mla_decode", "256 MLA decodes, ctx ~ U[1024, 32768], 16 q heads over one shared 512+64 latent record "
        "per token (bf16 or fp8 latent cache), paged KV (64)",
        0, 0, 16, 1, 576, 512, "bf16", "paged", seed=606,
        decode_requests=256, decode_ctx=(1024, 32768), scale_dim=192),
    # absorbed MLA chunked prefill: a 128K-token prompt in 8192-token chunks, 16 q heads attending to the
    # shared latent records (bf16 latent cache)
    "mla_prefill": Workload(
        "mla_prefill", "L=131072 as 16 chunks of 8192, 16 q heads over one shared 512+64 latent record per "
        "token (bf16 latent cache), paged KV (64)",
        131072, 8192, 16, 1, 576, 512, "bf16", "paged", seed=707, sample_rows=512, scale_dim=192),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(shape, seed: int) -> np.ndarray:
    """iid N(0,1) float32 of ``shape``, deterministic in ``seed`` alone."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)
    n_slabs = max(1, math.ceil(n / SLAB))
    children = np.random.SeedSequence(seed).spawn(n_slabs)

    def fill(i):
        lo, hi = i * SLAB, min(n, (i + 1) * SLAB)
        np.random.default_rng(children[i]).standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if n_slabs == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n_slabs)))
    return out.reshape(shape)


def normal(shape, seed: int, dtype: str) -> torch.Tensor:
    """Host tensor of iid N(0,1) draws, float32 or rounded to bfloat16."""
    t = torch.from_numpy(normal_f32(shape, seed))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


def normal_device(shape, seed: int, dtype: str, device="cuda") -> torch.Tensor:
    """Device tensor of iid N(0,1) draws from torch's seeded device generator."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def to_oracle(t: torch.Tensor) -> np.ndarray:
    """Host numpy view for the oracle: float32 as is, bf16 as uint16 bit patterns."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def pool_size(needed_blocks: int) -> int:
    return max(1, math.ceil(1.25 * needed_blocks))


def block_table(needed_blocks: int, seed: int, pool_blocks: int | None = None) -> np.ndarray:
    """Seeded draw of ``needed_blocks`` distinct physical block ids (int32)."""
    pool = pool_size(needed_blocks) if pool_blocks is None else pool_blocks
    rng = np.random.default_rng(seed)
    return rng.choice(pool, size=needed_blocks, replace=False).astype(np.int32)


def context_lengths(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Seeded integers uniform on [lo, hi] (both ends included), int32."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=n, endpoint=True).astype(np.int32)


def batch_block_tables(kv_lens, seed: int):
    """Disjoint seeded blocks for every sequence of a batch: ([n, max_blocks] int32, pool_blocks)."""
    needed = [max(1, math.ceil(int(k) / BLOCK_SIZE)) for k in kv_lens]
    pool_blocks = pool_size(sum(needed))
    perm = block_table(sum(needed), seed, pool_blocks)
    tables = np.zeros((len(needed), max(needed) if needed else 1), dtype=np.int32)
    off = 0
    for s, nb in enumerate(needed):
        tables[s, :nb] = perm[off: off + nb]
        off += nb
    return tables, pool_blocks


def mla_record_seed(w: Workload, s: int) -> int:
    """Seed of sequence s's latent records (device draws: latents, then rotary parts)."""
    return w.seed * 1000 + 10 + s


def sample_rows(chunk_len: int, heads: int, n: int, seed: int):
    """Seeded (token, head) rows of one chunk; always includes the edge tokens."""
    rng = np.random.default_rng(seed)
    must = {0, chunk_len - 1}
    for tile in (64, 128):
        for b in range(tile, chunk_len, tile):
            must.update((b - 1, b))
    must = sorted(t for t in must if 0 <= t < chunk_len)
    if len(must) > n // 2:
        keep = rng.choice(len(must), size=n // 2, replace=False)
        must = sorted({must[i] for i in keep} | {0, chunk_len - 1})
    rest = max(0, n - len(must))
    toks = np.concatenate([np.asarray(must, dtype=np.int64),
                           rng.integers(0, chunk_len, size=rest, dtype=np.int64)])
    hds = rng.integers(0, heads, size=toks.shape[0], dtype=np.int64).astype(np.int32)
    return toks, hds


def chunk_seeds(w: Workload, k: int) -> int:
    """Seed of chunk k's queries; keys and values use ``w.seed + 1`` / ``+ 2``."""
    return w.seed * 1000 + 10 + k
