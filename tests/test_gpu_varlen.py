"""GPU parity of the mixed prefill + decode batch (varlen entry) against the fp64 oracle.

A batch mixes prefill chunks (many query tokens at an offset) with decode
requests (one query token, or a few, reading the whole cache), as in the
notes on "Revisiting Pipeline Parallelism for LLM Serving" (preliminaries).
Each sequence owns its own blocks of one shared paged pool; every output row
and every LSE value is compared with the oracle run on that sequence alone.
"""
import math

import numpy as np
import pytest
import torch

from chunked_prefill_causal_amd import _lib as L
from chunked_prefill_causal_amd import inputs

from gpu_common import BF16_TOL, LSE_TOL, Pool, build_batch, log, max_err, oracle_chunk, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def check_batch(q_lens, kv_lens, hq, hkv, d, dv, seed):
    pool, tables, cu, q_all, seqs = build_batch(q_lens, kv_lens, hq, hkv, d, dv, seed)
    scale = 1.0 / math.sqrt(d)
    out, lse = L.chunk_attn_varlen(q_all.cuda(), pool.k, pool.v, tables, cu, kv_lens, scale, return_lse=True)
    worst, worst_lse = 0.0, 0.0
    for s, (q, k, v) in enumerate(seqs):
        if q_lens[s] == 0:
            continue
        ref, ref_lse = oracle_chunk(q, k, v, kv_lens[s] - q_lens[s], scale)
        worst = max(worst, max_err(out[cu[s]: cu[s + 1]], ref))
        worst_lse = max(worst_lse, max_err(lse[:, cu[s]: cu[s + 1]], ref_lse))
    log(f"varlen q_lens={q_lens[:6]}... kv_lens={kv_lens[:6]}...: max err {worst:.3e}, lse {worst_lse:.2e}")
    assert worst <= BF16_TOL and worst_lse <= LSE_TOL


def test_mixed_small():
    check_batch([200, 1, 1, 1, 1], [1300, 1, 64, 65, 3000], 32, 8, 128, 128, 5000)


@pytest.mark.parametrize("d,dv,hq,hkv", [(128, 128, 32, 8), (192, 128, 16, 16), (64, 64, 8, 2)])
def test_fp32_output(d, dv, hq, hkv):
    """out_dtype fp32: every row against the oracle at the plain bar (no bf16 store), and the bf16 output of
    the same batch equals the fp32 output rounded to bf16 bit for bit (one rounding of the same value)."""
    q_lens = [300, 1, 1, 3, 1, 0, 150]
    kv_lens = [1000, 77, 4100, 600, 1, 9, 150]
    pool, tables, cu, q_all, seqs = build_batch(q_lens, kv_lens, hq, hkv, d, dv, 5050 + d)
    scale = 1.0 / math.sqrt(d)
    log(f"varlen fp32 output d={d}/{dv} heads {hq}/{hkv}")
    out32, lse32 = L.chunk_attn_varlen(q_all.cuda(), pool.k, pool.v, tables, cu, kv_lens, scale,
                                       out_dtype=torch.float32, return_lse=True)
    out16, lse16 = L.chunk_attn_varlen(q_all.cuda(), pool.k, pool.v, tables, cu, kv_lens, scale, return_lse=True)
    assert out32.dtype == torch.float32 and out16.dtype == torch.bfloat16
    assert torch.equal(out32.to(torch.bfloat16).view(torch.int16), out16.view(torch.int16))
    assert torch.equal(lse32, lse16)
    worst = worst_lse = 0.0
    for s, (q, k, v) in enumerate(seqs):
        if q_lens[s] == 0:
            continue
        ref, ref_lse = oracle_chunk(q, k, v, kv_lens[s] - q_lens[s], scale)
        worst = max(worst, max_err(out32[cu[s]: cu[s + 1]], ref))
        worst_lse = max(worst_lse, max_err(lse32[:, cu[s]: cu[s + 1]], ref_lse))
    log(f"  max err {worst:.3e}, lse {worst_lse:.2e}")
    assert worst <= BF16_TOL and worst_lse <= LSE_TOL


def test_decode_only_ragged_contexts():
    rng = np.random.default_rng(3)
    kv = rng.integers(1, 5000, size=24).tolist()
    check_batch([1] * 24, kv, 32, 8, 128, 128, 5100)


def test_decode_contexts_at_tile_and_split_edges():
    """Contexts at, one below and one above 64-key tiles and 256-key splits (the split length
    a small batch gets), so a split may hold a single key or end exactly on a tile."""
    kv = [1, 63, 64, 65, 127, 128, 255, 256, 257, 511, 512, 513, 768, 769, 1023, 1024]
    check_batch([1] * len(kv), kv, 32, 8, 128, 128, 5150)
    check_batch([1] * len(kv), kv, 16, 16, 64, 64, 5160)


def test_short_multi_token_rows_take_decode_path():
    """q_len * group <= 32 rides the split-KV path with a causal mask inside the group."""
    check_batch([2, 8, 3, 40], [900, 2100, 3, 600], 16, 4, 128, 128, 5200)


def test_mixed_mha_d64_and_mla_dims():
    check_batch([130, 1, 1], [500, 777, 64], 8, 8, 64, 64, 5300)
    check_batch([100, 1, 1], [300, 1000, 129], 4, 4, 192, 128, 5400)


def test_empty_sequences_are_skipped():
    check_batch([0, 1, 0, 70, 1], [10, 10, 5, 100, 2000], 8, 2, 128, 128, 5500)


def test_lse_and_out_rows_untouched_outside_batch_rows():
    """The output of a batch holds exactly total_q rows; nothing else is written."""
    pool, tables, cu, q_all, seqs = build_batch([1, 1], [100, 200], 8, 2, 128, 128, 5600)
    out = torch.full((4, 8, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    L.chunk_attn_varlen(q_all.cuda(), pool.k, pool.v, tables, cu, [100, 200], 0.1, out=out[:2])
    assert torch.all(out[2:] == 7.0)


def test_most_sequences():
    """65535 sequences, the most the entry takes: one 300-token chunk at past 700 and 65534 decodes of 1-100
    keys, 4 query heads over 1 KV head, d 128.  The device-side plan's threads own many sequences each and
    the decode and merge grids span every sequence.  The batch's K/V and queries are drawn in one pass each
    (sequence s takes the next kv_lens[s] tokens); the chunk, every 257th decode and the last ones are checked
    against the oracle."""
    rng = np.random.default_rng(7100)
    n, hq, hkv, d = 65535, 4, 1, 128
    kv = rng.integers(1, 101, size=n).astype(np.int64)
    kv[0], kv[-1] = 1000, 1
    q_lens = np.ones(n, dtype=np.int64)
    q_lens[0] = 300
    needed = (kv + 63) // 64
    pool_blocks = inputs.pool_size(int(needed.sum()))
    perm = inputs.block_table(int(needed.sum()), 7100, pool_blocks)
    first = np.concatenate([[0], np.cumsum(needed)])
    tables = np.zeros((n, int(needed.max())), dtype=np.int32)
    for s in range(n):
        tables[s, : needed[s]] = perm[first[s]: first[s + 1]]
    tables_d = torch.from_numpy(tables).cuda()
    tok0 = np.concatenate([[0], np.cumsum(kv)])
    k_all = inputs.normal((int(kv.sum()), hkv, d), 7101, "bf16")
    v_all = inputs.normal((int(kv.sum()), hkv, d), 7102, "bf16")
    pool = Pool(pool_blocks, hkv, d, d, torch.bfloat16)
    k_dev, v_dev = k_all.cuda(), v_all.cuda()
    for s in range(n):
        L.chunkattn_kv_append(k_dev[tok0[s]: tok0[s + 1]], v_dev[tok0[s]: tok0[s + 1]], 0, tables_d[s], pool.k, pool.v)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q_all = inputs.normal((int(cu[-1]), hq, d), 7103, "bf16")
    scale = 1.0 / math.sqrt(d)
    log(f"varlen: {n} sequences, {int(kv.sum())} cached tokens, {int(cu[-1])} query rows")
    out, lse = L.chunk_attn_varlen(q_all.cuda(), pool.k, pool.v, tables_d, cu, kv.tolist(), scale, return_lse=True)
    torch.cuda.synchronize()
    worst, worst_lse = 0.0, 0.0
    for s in [0] + list(range(1, n, 257)) + [n - 2, n - 1]:
        q = q_all[cu[s]: cu[s + 1]]
        k, v = k_all[tok0[s]: tok0[s + 1]], v_all[tok0[s]: tok0[s + 1]]
        ref, ref_lse = oracle_chunk(q, k, v, int(kv[s] - q_lens[s]), scale)
        worst = max(worst, max_err(out[cu[s]: cu[s + 1]], ref))
        worst_lse = max(worst_lse, max_err(lse[:, cu[s]: cu[s + 1]], ref_lse))
    log(f"  sampled sequences: max err {worst:.3e}, lse {worst_lse:.2e}")
    assert worst <= BF16_TOL and worst_lse <= LSE_TOL


@pytest.mark.parametrize("seed", [7001, 7002, 7003, 7004])
def test_random_mixed_batches(seed):
    """Seeded random batches: 4-12 sequences mixing prefill chunks (q_len up to 300) with decode
    requests (q_len 1-4), contexts 1..4000 with q_len <= kv_len, a random GQA ratio and head-dim pair."""
    rng = np.random.default_rng(seed)
    hq, hkv = [(32, 8), (16, 16), (8, 1), (12, 4)][seed % 4]
    d, dv = [(128, 128), (64, 64), (192, 128), (128, 128)][(seed // 2) % 4]
    n = int(rng.integers(4, 13))
    q_lens, kv_lens = [], []
    for _ in range(n):
        kv = int(rng.integers(1, 4001))
        q = int(rng.integers(1, 5)) if rng.random() < 0.6 else int(rng.integers(5, 301))
        q_lens.append(min(q, kv))
        kv_lens.append(kv)
    log(f"random batch seed {seed}: heads {hq}/{hkv}, d {d}/{dv}, q_lens {q_lens}, kv_lens {kv_lens}")
    check_batch(q_lens, kv_lens, hq, hkv, d, dv, seed)


def test_co_scheduled_calls_on_two_streams_match_serial_runs():
    """Two mixed batches large enough to run co-scheduled (a 512-token chunk at 4096 beside 48 decodes of
    2048 keys: the prefill part on one half of the GPU, the decode part on the other) are issued back to
    back on two streams, so they share the library's co-scheduling streams and events.  Each result must
    equal that batch run alone, bit for bit, on three repetitions."""
    scale = 1.0 / math.sqrt(128)
    q_lens, kv_lens = [512] + [1] * 48, [4608] + [2048] * 48
    batches = []
    for seed in (5700, 5800):
        pool, tables, cu, q_all, _ = build_batch(q_lens, kv_lens, 32, 8, 128, 128, seed)
        batches.append((pool, tables, cu, q_all.cuda()))
    run = lambda b, stream=None: L.chunk_attn_varlen(b[3], b[0].k, b[0].v, b[1], b[2], kv_lens, scale,
                                                     return_lse=True, stream=stream)
    alone = [run(b) for b in batches]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        got = []
        for b, st in zip(batches, streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                got.append(run(b, st))
        torch.cuda.synchronize()
        for (o, l), (o_ref, l_ref) in zip(got, alone):
            assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(l, l_ref)
        log(f"two co-scheduled batches on two streams, repetition {rep}: bitwise equal to the serial runs")
