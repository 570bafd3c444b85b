"""Parity at full workload sizes, in the launch configuration bench.py times.

Each workload runs every chunk of its prompt (or its whole mixed batch)
through the C ABI with default options (the library picks its own split
count), and seeded sampled rows are compared with the fp64 oracle, which
reads the same inputs copied to the host.  The sample always includes each
chunk's first and last token and tokens on both sides of tile boundaries.

Row counts per chunk: 4096 for the 32K, 128K and 512K MLA-shaped prompts
(the last as its workload states), 512 for the 128K MLA latent prompt (from
both cache formats), and every row of the mixed batch: all 8192 decode rows
and all 65536 rows of its 2048-token prefill chunk.  The
fp64 oracle needs a few CPU-minutes on 16 host cores for all of it.
"""
import math

import numpy as np
import pytest
import torch

from chunked_prefill_causal_amd import _lib as L
from chunked_prefill_causal_amd import inputs

from gpu_common import BF16_TOL, LSE_TOL, log, max_err, oracle_rows, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def run_prompt(name, rows_per_chunk):
    w = inputs.WORKLOADS[name]
    n, hq, hkv, d, dv = w.seq_len, w.heads, w.kv_heads, w.head_dim, w.head_dim_v
    log(f"{name}: generating {n} tokens of K/V on the device")
    k = inputs.normal_device((n, hkv, d), w.seed + 1, "bf16")
    v = inputs.normal_device((n, hkv, dv), w.seed + 2, "bf16")
    needed = math.ceil(n / 64)
    table = torch.from_numpy(inputs.block_table(needed, w.seed + 3)).cuda()
    kp, vp = L.paged_pool(inputs.pool_size(needed), hkv, d, dv, torch.bfloat16)
    kp.fill_(float("nan"))
    vp.fill_(float("nan"))
    L.chunkattn_kv_append(k, v, 0, table, kp, vp)
    k_host, v_host = k.cpu(), v.cpu()
    del k, v
    worst = worst_lse = 0.0
    for c in range(w.n_chunks):
        past = c * w.chunk_len
        q = inputs.normal_device((w.chunk_len, hq, d), inputs.chunk_seeds(w, c), "bf16")
        out, lse = L.chunk_prefill_attn(q, kp, vp, past, w.scale, kv_layout="paged", block_table=table,
                                        return_lse=True)
        tok, head = inputs.sample_rows(w.chunk_len, hq, rows_per_chunk, w.seed * 11 + c)
        ti, hi = torch.from_numpy(tok).cuda(), torch.from_numpy(head.astype(np.int64)).cuda()
        got, got_lse = out[ti, hi], lse[hi, ti]
        ref, ref_lse = oracle_rows(q.cpu(), k_host[: past + w.chunk_len], v_host[: past + w.chunk_len], past,
                                   w.scale, tok, head)
        e, el = max_err(got, ref), max_err(got_lse, ref_lse)
        worst, worst_lse = max(worst, e), max(worst_lse, el)
        log(f"{name} chunk {c} (past {past}): {len(tok)} rows, max err {e:.3e}, lse err {el:.2e}")
    assert worst <= BF16_TOL and worst_lse <= LSE_TOL


def test_gqa_32k_all_chunks():
    run_prompt("gqa_32k", 4096)


def test_gqa_128k_all_chunks():
    run_prompt("gqa_128k", 4096)


def test_mla_512k_all_chunks():
    run_prompt("mla_512k", 4096)


def test_mla_prefill_all_chunks():
    """The 128K latent prompt (16 chunks of 8192, 16 heads) over both cache formats, as the benchmark runs it:
    the whole prompt's records are written first into a 0xFF-poisoned pool, every chunk runs, and sampled rows
    of each chunk are compared with the oracle on the records the prefill computes with (bf16, or the fp8
    records staged as bf16(code x scale))."""
    from oracle import mla
    w = inputs.WORKLOADS["mla_prefill"]
    needed = math.ceil(w.seq_len / 64)
    table = torch.from_numpy(inputs.block_table(needed, w.seed + 3)).cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(inputs.mla_record_seed(w, 0))
    lat = torch.randn((w.seq_len, L.MLA_LATENT), generator=gen, device="cuda").to(torch.bfloat16)
    rope = torch.randn((w.seq_len, L.MLA_ROPE), generator=gen, device="cuda").to(torch.bfloat16)
    lat_bits = lat.cpu().view(torch.int16).numpy().view(np.uint16)
    rope_bits = rope.cpu().view(torch.int16).numpy().view(np.uint16)
    worst = worst_lse = 0.0
    for fmt_name, fmt in (("bf16", L.CA_MLA_BF16), ("fp8", L.CA_MLA_FP8)):
        pool = L.mla_pool(inputs.pool_size(needed), fmt)
        pool.fill_(0xFF)
        L.chunkattn_mla_kv_append(lat, rope, 0, table, pool, fmt)
        recs = (mla.records(lat_bits, rope_bits, "bf16") if fmt_name == "bf16"
                else mla.fp8_staged_records(lat_bits, rope_bits))
        for c in range(w.n_chunks):
            past = c * w.chunk_len
            q = inputs.normal_device((w.chunk_len, w.heads, w.head_dim), inputs.chunk_seeds(w, c), "bf16")
            out, lse = L.chunk_mla_prefill(q, pool, fmt, table, past, w.scale, return_lse=True)
            tok, head = inputs.sample_rows(w.chunk_len, w.heads, w.sample_rows, w.seed * 11 + c)
            ti, hi = torch.from_numpy(tok).cuda(), torch.from_numpy(head.astype(np.int64)).cuda()
            q_bits = q.cpu().view(torch.int16).numpy().view(np.uint16)
            ref, ref_lse = mla.prefill(q_bits, recs, past, w.scale, tok, head)
            e, el = max_err(out[ti, hi], ref), max_err(lse[hi, ti], ref_lse)
            worst, worst_lse = max(worst, e), max(worst_lse, el)
            log(f"mla_prefill {fmt_name} chunk {c} (past {past}): {len(tok)} rows, max err {e:.3e}, lse err {el:.2e}")
        del pool
        torch.cuda.empty_cache()
    assert worst <= BF16_TOL and worst_lse <= LSE_TOL


def test_mixed_batch_full_size():
    w = inputs.WORKLOADS["mixed"]
    hq, hkv, d, dv = w.heads, w.kv_heads, w.head_dim, w.head_dim_v
    dec = inputs.context_lengths(w.decode_requests, w.decode_ctx[0], w.decode_ctx[1], w.seed + 7)
    q_lens = [w.chunk_len] + [1] * w.decode_requests
    kv_lens = [w.prefill_past + w.chunk_len] + dec.tolist()
    needed = [math.ceil(x / 64) for x in kv_lens]
    pool_blocks = inputs.pool_size(sum(needed))
    perm = inputs.block_table(sum(needed), w.seed + 8, pool_blocks)
    tables = np.zeros((len(kv_lens), max(needed)), dtype=np.int32)
    off = 0
    for s, nb in enumerate(needed):
        tables[s, :nb] = perm[off: off + nb]
        off += nb
    tables = torch.from_numpy(tables).cuda()
    kp, vp = L.paged_pool(pool_blocks, hkv, d, dv, torch.bfloat16)
    kp.fill_(float("nan"))
    vp.fill_(float("nan"))
    log(f"mixed: {len(kv_lens)} sequences, {sum(kv_lens)} cached tokens")
    kv_host = []
    for s, n in enumerate(kv_lens):
        kk = inputs.normal_device((n, hkv, d), w.seed + 100 + 2 * s, "bf16")
        vv = inputs.normal_device((n, hkv, dv), w.seed + 101 + 2 * s, "bf16")
        L.chunkattn_kv_append(kk, vv, 0, tables[s], kp, vp)
        kv_host.append((kk.cpu(), vv.cpu()))
    q_all = inputs.normal_device((sum(q_lens), hq, d), w.seed + 9, "bf16")
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    out, lse = L.chunk_attn_varlen(q_all, kp, vp, tables, cu, kv_lens, w.scale, return_lse=True)
    q_host = q_all.cpu()
    # every decode row
    worst = worst_lse = 0.0
    for s in range(1, len(kv_lens)):
        row = cu[s]
        ref, ref_lse = oracle_rows(q_host[row: row + 1], kv_host[s][0], kv_host[s][1], kv_lens[s] - 1, w.scale,
                                   np.zeros(hq, np.int64), np.arange(hq, dtype=np.int32))
        worst = max(worst, max_err(out[row], ref))
        worst_lse = max(worst_lse, max_err(lse[:, row], ref_lse))
    log(f"mixed: 256 decode requests x {hq} heads, max err {worst:.3e}, lse err {worst_lse:.2e}")
    # every (token, head) row of the prefill chunk
    tok = np.repeat(np.arange(w.chunk_len, dtype=np.int64), hq)
    head = np.tile(np.arange(hq, dtype=np.int32), w.chunk_len)
    ref, ref_lse = oracle_rows(q_host[: w.chunk_len], kv_host[0][0], kv_host[0][1], w.prefill_past, w.scale,
                               tok, head)
    ti, hi = torch.from_numpy(tok).cuda(), torch.from_numpy(head.astype(np.int64)).cuda()
    e, el = max_err(out[ti, hi], ref), max_err(lse[hi, ti], ref_lse)
    log(f"mixed: prefill chunk, all {len(tok)} rows, max err {e:.3e}, lse err {el:.2e}")
    assert max(worst, e) <= BF16_TOL and max(worst_lse, el) <= LSE_TOL
