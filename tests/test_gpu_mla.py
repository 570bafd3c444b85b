"""GPU parity of MLA latent (absorbed) decode and of the latent cache write,
against the fp64 oracle (oracle/mla.py).

"02 · 并行策略与 PP 切分 — GLM5.3 CyberSec W4A16" deployment notes §1, §4:
one latent record per token shared by every query head, 1152 B in bf16 or
656 B in the fp8 latent format.

* The cache write is compared byte for byte with the layout the header states,
  packed here on the host; fp8 codes and scales must equal the oracle's
  quantisation exactly, and bytes the write does not own must be untouched.
* Decode runs on pools packed on the host (so it does not lean on the write
  kernel), poisoned with 0xFF (NaN in bf16, in e4m3 and in the fp32 scales)
  outside the records that exist: no output may see them.  Every output value
  and LSE is compared with the oracle.
* The decode-batch workload (256 requests, contexts uniform in [1024, 32768],
  16 query heads) is filled by the write kernel and checked on sampled
  sequences, in the launch configuration the benchmark times.
Softmax scale 1/sqrt(192), the expanded head's 128 no-rope + 64 rope values.
"""
import math

import numpy as np
import pytest
import torch

from chunked_prefill_causal_amd import _lib as L
from chunked_prefill_causal_amd import inputs
import oracle
from oracle import mla

from gpu_common import BF16_TOL, LSE_TOL, log, max_err, require_gpu

pytestmark = pytest.mark.gpu

FMTS = {"bf16": L.CA_MLA_BF16, "fp8": L.CA_MLA_FP8}
SCALE = 1.0 / math.sqrt(192)
POISON = 0xFF


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def byte_offsets(fmt: str, table: np.ndarray, positions: np.ndarray):
    """Flat pool byte offsets of each position's (latent or codes, scales, rotary) bytes."""
    bb = L.chunkattn_mla_block_bytes(FMTS[fmt])
    base = table[positions // 64].astype(np.int64) * bb + (positions % 64) * 16
    if fmt == "bf16":                      # [72 runs][64 tokens][16 B]: record byte j in run j // 16
        j = np.arange(1152)
        rec = base[:, None] + (j // 16) * 1024 + j % 16
        return rec[:, :1024], None, rec[:, 1024:]
    # fp8: halves of 32 tokens, each codes [32 runs][32][16 B], scales [32][16 B], rotary [8 runs][32][16 B]
    half = table[positions // 64].astype(np.int64) * bb + ((positions % 64) // 32) * 20992
    u = positions % 32
    j = np.arange(512)
    codes = half[:, None] + ((j // 16) * 32 + u[:, None]) * 16 + j % 16
    scales = half[:, None] + 16384 + u[:, None] * 16 + np.arange(16)
    j = np.arange(128)
    rope = half[:, None] + 16896 + ((j // 16) * 32 + u[:, None]) * 16 + j % 16
    return codes, scales, rope


def pack(pool: np.ndarray, fmt: str, table: np.ndarray, lat_bits, rope_bits, start: int = 0) -> None:
    """Write records of positions start.. into a flat host pool, as the header lays them out."""
    n = lat_bits.shape[0]
    lat_off, sc_off, rope_off = byte_offsets(fmt, table, np.arange(start, start + n))
    pool[rope_off] = rope_bits.view(np.uint8).reshape(n, 128)
    if fmt == "bf16":
        pool[lat_off] = lat_bits.view(np.uint8).reshape(n, 1024)
    else:
        codes, scales = mla.quantize_latent(inputs_f32(lat_bits))
        pool[lat_off] = codes
        pool[sc_off] = scales.view(np.uint8).reshape(n, 16)


def inputs_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def new_pool(fmt, num_blocks, fill):
    return torch.full((num_blocks, L.chunkattn_mla_block_bytes(FMTS[fmt])), fill, dtype=torch.uint8, device="cuda")


# ------------------------------------------------------------- cache write
def special_latents(n, seed):
    """Seeded latents with the quantiser's corner cases in the first rows."""
    lat = inputs.normal((n, 512), seed, "f32").numpy() * np.float32(2.0)
    lat[0, 128:256] = 0.0                                   # all-zero group: scale 1
    lat[1, 256:384] = -0.0                                  # all negative zero: codes 0x80
    lat[2, 0:128] *= np.float32(1e-30)                      # tiny group
    lat[2, 5] = np.float32(3e-28)
    lat[3, :] *= np.float32(1e30)                           # huge values
    lat[4, 0:128] = 1.0                                     # amax 448 -> scale 1; exact midpoints
    lat[4, 0] = 448.0
    lat[4, 1:8] = [1.0625, 1.1875, 432.0, 3 * 2.0 ** -10, 2.0 ** -10, -1.0625, -432.0]
    lat[5, 384:512] = np.linspace(-7, 7, 128, dtype=np.float32)
    lat[6, 0:128] = 0.0                                     # scale 1; subnormal codes and their midpoints
    lat[6, 0] = 448.0
    lat[6, 1:12] = np.array([1, 1.5, 2, 2.5, 3, 5, 6.5, 7, 7.5, -1.5, -0.5], dtype=np.float32) * 2.0 ** -9
    t = torch.from_numpy(lat).to(torch.bfloat16)
    return t


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_append_layout_bitexact(fmt):
    start, n, cap = 37, 230, 300
    needed = math.ceil(cap / 64)
    nb = inputs.pool_size(needed)
    table = inputs.block_table(needed, 31, nb)
    lat = special_latents(n, 40)
    rope = inputs.normal((n, 64), 41, "bf16")
    log(f"mla append fmt={fmt} start={start} n={n} blocks={nb}")
    pool = new_pool(fmt, nb, 0xAB)
    L.chunkattn_mla_kv_append(lat.cuda(), rope.cuda(), start, torch.from_numpy(table).cuda(), pool, FMTS[fmt])
    got = pool.cpu().numpy().reshape(-1)
    want = np.full(got.shape, 0xAB, dtype=np.uint8)
    pack(want, fmt, table, bits(lat), bits(rope), start)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}: got {got[bad[:8]]} want {want[bad[:8]]}"


def test_append_two_calls_fill_one_sequence():
    """A prefill chunk then one decode token: the second call lands after the first."""
    table = inputs.block_table(3, 32, 5)
    t_d = torch.from_numpy(table).cuda()
    lat = inputs.normal((129, 512), 42, "bf16")
    rope = inputs.normal((129, 64), 43, "bf16")
    for fmt in ("bf16", "fp8"):
        log(f"mla append two calls fmt={fmt}")
        pool = new_pool(fmt, 5, 0)
        L.chunkattn_mla_kv_append(lat[:128].cuda(), rope[:128].cuda(), 0, t_d, pool, FMTS[fmt])
        L.chunkattn_mla_kv_append(lat[128:].cuda(), rope[128:].cuda(), 128, t_d, pool, FMTS[fmt])
        want = np.zeros(pool.numel(), dtype=np.uint8)
        pack(want, fmt, table, bits(lat), bits(rope))
        assert np.array_equal(pool.cpu().numpy().reshape(-1), want)


# ------------------------------------------------------------------ decode
def build_batch(fmt, kv_lens, heads, seed):
    n = len(kv_lens)
    needed = [math.ceil(k / 64) for k in kv_lens]
    nb = inputs.pool_size(sum(needed))
    perm = inputs.block_table(sum(needed), seed, nb)
    tables = np.zeros((n, max(needed)), dtype=np.int32)
    host = np.full(nb * L.chunkattn_mla_block_bytes(FMTS[fmt]), POISON, dtype=np.uint8)
    seqs, off = [], 0
    for s, kv in enumerate(kv_lens):
        tables[s, : needed[s]] = perm[off: off + needed[s]]
        off += needed[s]
        lat = bits(inputs.normal((kv, 512), seed + 7 * s + 1, "bf16"))
        rope = bits(inputs.normal((kv, 64), seed + 7 * s + 2, "bf16"))
        pack(host, fmt, tables[s], lat, rope)
        seqs.append((lat, rope))
    q = inputs.normal((n, heads, 576), seed + 5, "bf16")
    pool = torch.from_numpy(host.reshape(nb, -1)).cuda()
    return pool, torch.from_numpy(tables).cuda(), q, seqs


def build_batch_flat(fmt, kv_lens, heads, seed):
    """build_batch for many short sequences: one draw for all the batch's records (sequence s takes the next
    kv_lens[s] of them) and one packing pass, the block of each token looked up through its own table row."""
    n = len(kv_lens)
    kv = np.asarray(kv_lens, dtype=np.int64)
    needed = (kv + 63) // 64
    nb = inputs.pool_size(int(needed.sum()))
    perm = inputs.block_table(int(needed.sum()), seed, nb)
    tables = np.zeros((n, int(needed.max())), dtype=np.int32)
    first = np.concatenate([[0], np.cumsum(needed)])
    for s in range(n):
        tables[s, : needed[s]] = perm[first[s]: first[s + 1]]
    total = int(kv.sum())
    lat = bits(inputs.normal((total, 512), seed + 1, "bf16"))
    rope = bits(inputs.normal((total, 64), seed + 2, "bf16"))
    seq_of = np.repeat(np.arange(n), kv)
    tok0 = np.concatenate([[0], np.cumsum(kv)])
    pos = np.arange(total) - tok0[seq_of]
    # byte_offsets through a per-token table: entry t of `flat` is the block of token t's position
    flat = tables[seq_of, pos // 64]
    host = np.full(nb * L.chunkattn_mla_block_bytes(FMTS[fmt]), POISON, dtype=np.uint8)
    lat_off, sc_off, rope_off = byte_offsets(fmt, flat, pos % 64 + 64 * np.arange(total))
    host[rope_off] = rope.view(np.uint8).reshape(total, 128)
    if fmt == "bf16":
        host[lat_off] = lat.view(np.uint8).reshape(total, 1024)
    else:
        codes, scales = mla.quantize_latent(inputs_f32(lat))
        host[lat_off] = codes
        host[sc_off] = scales.view(np.uint8).reshape(total, 16)
    seqs = [(lat[tok0[s]: tok0[s + 1]], rope[tok0[s]: tok0[s + 1]]) for s in range(n)]
    q = inputs.normal((n, heads, 576), seed + 5, "bf16")
    pool = torch.from_numpy(host.reshape(nb, -1)).cuda()
    return pool, torch.from_numpy(tables).cuda(), q, seqs


def bf16_half_ulp(x) -> np.ndarray:
    """Half the bf16 spacing at |x|: the most one round-to-nearest-even store can change x."""
    e = np.floor(np.log2(np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)))
    return 2.0 ** (e - 8)


def check_decode(fmt, kv_lens, heads, seed, sample=None, out_dtype=torch.bfloat16):
    """Every output against the oracle.  The batch always runs with fp32 output, held to the plain bar.  A
    bf16-output run must equal that fp32 output rounded once to bf16, bit for bit (the same value stored
    twice), so its error beyond the store's own rounding is the fp32 output's; it is also reported against
    the bar plus half a bf16 spacing (up to 0.0156 for |o| in [4, 8))."""
    pool, tables, q, seqs = (build_batch_flat if len(kv_lens) > 5000 else build_batch)(fmt, kv_lens, heads, seed)
    log(f"mla decode fmt={fmt} heads={heads} out={out_dtype} kv={list(kv_lens)[:12]} n={len(kv_lens)} seed={seed}")
    out32, lse32 = L.chunk_mla_decode(q.cuda(), pool, FMTS[fmt], tables, kv_lens, SCALE, return_lse=True,
                                      out_dtype=torch.float32)
    if out_dtype == torch.bfloat16:
        out16, lse16 = L.chunk_mla_decode(q.cuda(), pool, FMTS[fmt], tables, kv_lens, SCALE, return_lse=True)
        assert torch.equal(out32.to(torch.bfloat16).view(torch.int16), out16.view(torch.int16))
        assert torch.equal(lse32, lse16)
        out16 = out16.float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    out, lse = out32.cpu().numpy().astype(np.float64), lse32.cpu()
    assert np.all(np.isfinite(out)), "non-finite GPU output"
    qb = bits(q)
    worst = worst_excess = worst_lse = 0.0
    for s in (range(len(kv_lens)) if sample is None else sample):
        ref, ref_lse = mla.decode(qb[s], mla.records(*seqs[s], fmt), SCALE)
        worst = max(worst, float(np.abs(out[s] - ref).max()))
        if out_dtype == torch.bfloat16:
            err = np.abs(out16[s] - ref)
            # the pre-store value rounds to out within its own binade, which |ref| or |out| bounds from above
            store = bf16_half_ulp(np.maximum(np.abs(ref), np.abs(out16[s])))
            worst_excess = max(worst_excess, float((err - store).max()))
        worst_lse = max(worst_lse, max_err(lse[:, s], ref_lse))
    log(f"  fp32 output max abs err {worst:.3e}  bf16 output beyond its store's rounding {worst_excess:.3e}  "
        f"lse {worst_lse:.3e}")
    assert worst <= BF16_TOL and worst_excess <= BF16_TOL and worst_lse <= LSE_TOL


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_decode_ragged_contexts(fmt):
    # every step-tail length class: 1 key, one short of / exactly / one past 32 and 64, long
    check_decode(fmt, [1, 31, 32, 33, 63, 64, 65, 100, 1000, 4097], 16, 100)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("heads", [32, 128])
def test_decode_more_heads(fmt, heads):
    check_decode(fmt, [7, 129, 2000, 3333], heads, 200 + heads)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_decode_most_heads(fmt):
    # 1024 heads = 64 head blocks: the plan keeps its minimum of 8 units per head block
    check_decode(fmt, [1, 77, 300], 1024, 250)


def test_decode_most_sequences():
    # 65535 sequences, the most the entry takes, with 1-8 keys each: the plan kernel's threads own 64
    # sequences each, a work unit spans ~130 of them, and the merge grid is 65535 x 16 workgroups;
    # every 199th sequence and the last ones against the oracle
    rng = np.random.default_rng(520)
    kv = rng.integers(1, 9, size=65535).tolist()
    kv[0], kv[-1] = 8, 1
    sample = list(range(0, 65535, 199)) + [65533, 65534]
    check_decode("fp8", kv, 16, 520, sample=sample, out_dtype=torch.float32)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_decode_units_spanning_many_blocks(fmt):
    # 1024 heads keep the plan at 8 units per head block, so the 70000-key context is cut into
    # segments of ~274 steps (up to 138 cache blocks): their block ids fill all three of the
    # kernel's lane-indexed id registers
    check_decode(fmt, [70000, 3, 65], 1024, 260)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_decode_many_splits(fmt):
    # one long context among short ones: the plan gives it many splits
    check_decode(fmt, [40000, 5, 70, 300], 16, 300)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16out", "f32out"])
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_decode_thousands_of_short_sequences(fmt, out_dtype):
    # 3000 sequences: the plan kernel's threads each own several sequences, and
    # a work unit spans many short sequences (one partial per segment).  Short
    # contexts give outputs up to |o| ~ 5, where one bf16 store alone may err
    # by 0.0156: fp32 output shows the kernel itself within the bar.
    rng = np.random.default_rng(500)
    kv = rng.integers(1, 200, size=3000).tolist()
    kv[0], kv[1], kv[-1] = 1, 33, 64
    check_decode(fmt, kv, 16, 500, out_dtype=out_dtype)


def test_decode_rejects_unsupported_heads_on_device():
    q = torch.zeros((1, 8, 576), dtype=torch.bfloat16, device="cuda")
    pool = new_pool("bf16", 1, 0)
    with pytest.raises(L.ChunkAttnError):
        L.chunk_mla_decode(q, pool, L.CA_MLA_BF16, torch.zeros((1, 1), dtype=torch.int32, device="cuda"), [10], SCALE)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_decode_after_append_end_to_end(fmt):
    """Records written by the cache-write kernel (prefix, then one decode token) and read by decode."""
    kv = [700, 65, 1]
    needed = [math.ceil(k / 64) for k in kv]
    nb = inputs.pool_size(sum(needed))
    perm = inputs.block_table(sum(needed), 400, nb)
    tables = np.zeros((3, max(needed)), dtype=np.int32)
    pool = new_pool(fmt, nb, POISON)
    recs, off = [], 0
    for s, n in enumerate(kv):
        tables[s, : needed[s]] = perm[off: off + needed[s]]
        off += needed[s]
        lat = inputs.normal((n, 512), 410 + s, "bf16")
        rope = inputs.normal((n, 64), 420 + s, "bf16")
        t_d = torch.from_numpy(tables[s]).cuda()
        log(f"mla append+decode fmt={fmt} seq={s} n={n}")
        if n > 1:
            L.chunkattn_mla_kv_append(lat[:-1].cuda(), rope[:-1].cuda(), 0, t_d, pool, FMTS[fmt])
        L.chunkattn_mla_kv_append(lat[-1:].cuda(), rope[-1:].cuda(), n - 1, t_d, pool, FMTS[fmt])
        recs.append(mla.records(bits(lat), bits(rope), fmt))
    q = inputs.normal((3, 16, 576), 430, "bf16")
    out, lse = L.chunk_mla_decode(q.cuda(), pool, FMTS[fmt], torch.from_numpy(tables).cuda(), kv, SCALE,
                                  return_lse=True)
    out, lse = out.cpu(), lse.cpu()
    for s in range(3):
        ref, ref_lse = mla.decode(bits(q)[s], recs[s], SCALE)
        assert max_err(out[s], ref) <= BF16_TOL
        assert max_err(lse[:, s], ref_lse) <= LSE_TOL


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_decode_batch_workload_sampled(fmt):
    """The benchmark's MLA decode batch (same seeds, tables and launch): sampled sequences vs the oracle."""
    w = inputs.WORKLOADS["mla_decode"]
    kv = inputs.context_lengths(w.decode_requests, w.decode_ctx[0], w.decode_ctx[1], w.seed)
    tables, nb = inputs.batch_block_tables(kv, w.seed + 1)
    tables_d = torch.from_numpy(tables).cuda()
    pool = new_pool(fmt, nb, POISON)
    log(f"mla workload fmt={fmt}: filling {int(kv.sum())} tokens")
    gen = torch.Generator(device="cuda")
    n = w.decode_requests
    sample = sorted({0, n - 1, int(np.argmax(kv)), int(np.argmin(kv)), 17, 130})
    kept = {}
    for s in range(n):
        gen.manual_seed(inputs.mla_record_seed(w, s))
        lat = torch.randn((int(kv[s]), 512), generator=gen, device="cuda").to(torch.bfloat16)
        rope = torch.randn((int(kv[s]), 64), generator=gen, device="cuda").to(torch.bfloat16)
        L.chunkattn_mla_kv_append(lat, rope, 0, tables_d[s], pool, FMTS[fmt])
        if s in sample:
            kept[s] = (bits(lat.cpu()), bits(rope.cpu()))
    q = inputs.normal_device((n, w.heads, w.head_dim), w.seed + 2, "bf16")
    assert w.scale == SCALE
    log(f"mla workload fmt={fmt}: decode")
    out, lse = L.chunk_mla_decode(q, pool, FMTS[fmt], tables_d, kv, w.scale, return_lse=True)
    out, lse, qb = out.cpu(), lse.cpu(), bits(q.cpu())
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    worst = worst_lse = 0.0
    for s in sample:
        ref, ref_lse = mla.decode(qb[s], mla.records(*kept[s], fmt), SCALE)
        worst = max(worst, max_err(out[s], ref))
        worst_lse = max(worst_lse, max_err(lse[:, s], ref_lse))
    log(f"  sampled {sample}: max abs err {worst:.3e} lse {worst_lse:.3e}")
    assert worst <= BF16_TOL and worst_lse <= LSE_TOL


# ------------------------------------------------------------- chunked prefill
# VPP review §2.3: a prompt is cut into chunks; each chunk's records are appended
# to the cache, then its queries attend to every earlier record and causally to
# the chunk itself.  Pools start as 0xFF (NaN) everywhere: unowned blocks, block
# tails and the positions of later chunks must never reach an output.
def prompt_records(n, seed, rope_scale=None):
    """Latents and rotary parts of one prompt.  ``rope_scale(pos)`` multiplies the rotary parts: that moves
    the logits (and so the running maxima) while the values, the latents, stay N(0, 1)."""
    lat = inputs.normal((n, 512), seed, "f32")
    rope = inputs.normal((n, 64), seed + 1, "f32")
    if rope_scale is not None:
        rope = rope * torch.from_numpy(rope_scale(np.arange(n)).astype(np.float32))[:, None]
    return lat.to(torch.bfloat16), rope.to(torch.bfloat16)


def check_prefill(fmt, chunks, heads, seed, out_dtype=torch.bfloat16, rope_scale=None, sample=None):
    """Every compared row against the oracle on the records the prefill computes with: the bf16 records, or
    for an fp8 cache bf16(fp32(code x scale)).  For fp8 the LSE is also held to the exact fp8 records, within
    what that one rounding (2^-8 relative per key value) can move a logit: 2^-8 * scale * max_k sum |q| |k|."""
    n = sum(chunks)
    lat, rope = prompt_records(n, seed, rope_scale)
    if fmt == "bf16":
        recs, exact = mla.records(bits(lat), bits(rope), "bf16"), None
    else:
        recs, exact = mla.fp8_staged_records(bits(lat), bits(rope)), mla.records(bits(lat), bits(rope), "fp8")
    needed = math.ceil(n / 64)
    nb = inputs.pool_size(needed)
    table = torch.from_numpy(inputs.block_table(needed, seed + 2, nb)).cuda()
    pool = new_pool(fmt, nb, POISON)
    worst = worst_excess = worst_lse = worst_exact = 0.0
    past = 0
    for ci, c in enumerate(chunks):
        L.chunkattn_mla_kv_append(lat[past: past + c].cuda(), rope[past: past + c].cuda(), past, table, pool,
                                  FMTS[fmt])
        q = inputs.normal((c, heads, 576), seed + 10 + ci, "bf16")
        log(f"mla prefill fmt={fmt} heads={heads} out={out_dtype} chunk {ci}: past {past} len {c} seed {seed}")
        out, lse = L.chunk_mla_prefill(q.cuda(), pool, FMTS[fmt], table, past, SCALE, out_dtype=out_dtype,
                                       return_lse=True)
        torch.cuda.synchronize()
        out = out.float().cpu().numpy().astype(np.float64)
        lse = lse.cpu()
        assert np.all(np.isfinite(out)) and torch.isfinite(lse).all(), "non-finite GPU output"
        if sample is None:
            tok = np.repeat(np.arange(c, dtype=np.int64), heads)
            head = np.tile(np.arange(heads, dtype=np.int32), c)
        else:
            tok, head = inputs.sample_rows(c, heads, sample, seed * 7 + ci)
        ref, ref_lse = mla.prefill(bits(q), recs, past, SCALE, tok, head)
        got = out[tok, head]
        err = np.abs(got - ref)
        store = bf16_half_ulp(np.maximum(np.abs(ref), np.abs(got))) if out_dtype == torch.bfloat16 else 0.0
        worst = max(worst, float(err.max()))
        worst_excess = max(worst_excess, float((err - store).max()))
        worst_lse = max(worst_lse, max_err(lse[head, tok], ref_lse))
        if exact is not None:
            sel = np.random.default_rng(seed + ci).choice(len(tok), size=min(len(tok), 1024), replace=False)
            ts, hs = tok[sel], head[sel]
            _, ex_lse = mla.prefill(bits(q), exact, past, SCALE, ts, hs)
            qa = np.abs(oracle.bf16_bits_to_f64(bits(q))[ts, hs])
            dots = qa @ np.abs(exact[: past + c]).T
            dots[np.arange(past + c)[None, :] > (past + ts)[:, None]] = 0.0
            bound = 2.0 ** -8 * SCALE * dots.max(axis=1)
            dev = np.abs(lse[hs, ts].numpy().astype(np.float64) - ex_lse)
            worst_exact = max(worst_exact, float(dev.max()))
            assert np.all(dev <= LSE_TOL + bound), "LSE beyond the fp8 staging bound"
        past += c
    log(f"  max abs err {worst:.3e} (beyond the store's rounding {worst_excess:.3e})  lse {worst_lse:.3e}"
        + (f"  lse vs exact fp8 records {worst_exact:.3e}" if exact is not None else ""))
    assert worst_excess <= BF16_TOL and worst_lse <= LSE_TOL
    if out_dtype == torch.float32:
        assert worst <= BF16_TOL


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_prefill_multi_chunk_nan_poisoned(fmt):
    # chunk lengths: ragged, a single token, exactly one tile, several tiles; every row compared
    check_prefill(fmt, [130, 1, 64, 200, 95, 300], 16, 7100)


@pytest.mark.parametrize("fmt,heads,out_dtype", [("bf16", 32, torch.bfloat16), ("bf16", 48, torch.float32),
                                                 ("bf16", 128, torch.bfloat16), ("fp8", 64, torch.float32)],
                         ids=["bf16-h32", "bf16-h48-f32out", "bf16-h128", "fp8-h64-f32out"])
def test_prefill_more_heads(fmt, heads, out_dtype):
    check_prefill(fmt, [77, 250], heads, 7200 + heads, out_dtype=out_dtype)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_prefill_long_past_every_row(fmt):
    check_prefill(fmt, [5000, 700], 16, 7300)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_prefill_late_max_growth(fmt):
    # rotary parts grow with position, so a row's running maximum keeps rising and O is rescaled many times
    check_prefill(fmt, [600, 400], 16, 7400, rope_scale=lambda p: 1.0 + 12.0 * p / 1000.0)


def test_prefill_early_spike():
    # one early record with very large logits for many rows, then ordinary ones: the first tile fixes the maximum
    check_prefill("bf16", [40, 900], 16, 7500, rope_scale=lambda p: np.where(p == 3, 40.0, 1.0))
