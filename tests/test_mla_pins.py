"""Pins of the MLA oracle (oracle/mla.py) to facts outside itself.

* The e4m3 code table against the OCP 8-bit floating point format's
  definition (exponent bias 7, three mantissa bits, subnormals, largest normal
  448, the two NaN codes, no infinities): closed-form values of chosen codes.
* Encoding is nearest-value rounding with ties to the even code: checked by
  brute force over the whole finite table.
* Per-token bytes: "02 · 并行策略与 PP 切分 — GLM5.3 CyberSec W4A16" deployment
  notes §4 give 1152 B (bf16) and 656 B (fp8_ds_mla) per token and a 1.756x
  ratio; the record reading (512 latent + 64 rotary, one fp32 scale per 128
  latent values, rotary kept bf16) must give both.
* Absorbed decode against the expanded multi-head form: with per-head
  up-projections W_UK, W_UV, plain attention over keys [W_UK c ; rope] and
  values W_UV c equals W_UV applied to the latent-space output of the absorbed
  query [W_UK^T q_nope ; q_rope] (the identity that makes absorption exact).
  The expanded side runs through the package's general fp64 oracle with one KV
  head per query head, a different wiring from the shared-latent path.
* Special cases: one record, a zero query (uniform average, LSE = log L).
* Absorbed prefill of a chunk at past_len > 0: a zero query averages exactly
  the records 0 .. its position (LSE = log(position + 1)), so an off-by-one in
  the causal range or in past_len fails; the first position of a sequence
  returns record 0's latent; records after a row's position (or past the
  chunk) never change it; and the chunk equals the expanded multi-head form.
* fp8 records as the prefill stages them: values representable in bf16,
  within the bf16 rounding bound (2^-8 relative) of the exact code x scale,
  equal to it where the scale is a power of two, and nearest-even on a tie.
"""
import math

import numpy as np
import pytest

import oracle as orc
from oracle import mla


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16 (nearest even) as uint16 bit patterns."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


# ---------------------------------------------------------------- e4m3 table
def test_e4m3_table_closed_forms():
    v = mla.e4m3_values()
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and math.copysign(1, v[0x80]) == -1.0
    assert v[0x38] == 1.0                       # exponent field 7 = bias
    assert v[0x40] == 2.0
    assert v[0x3C] == 1.5
    assert v[0x7E] == 448.0                     # largest normal: 1.75 * 2^8
    assert v[0x7D] == 416.0
    assert v[0x08] == 2.0 ** -6                 # smallest normal
    assert v[0x07] == 7 * 2.0 ** -9             # largest subnormal
    assert v[0x01] == 2.0 ** -9                 # smallest subnormal
    assert v[0xBC] == -1.5
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(np.delete(v, [0x7F, 0xFF])).all()     # no infinities
    pos = v[:0x7F]
    assert (np.diff(pos) > 0).all()             # codes 0..0x7e increase strictly
    assert (v[0x80:0xFF] == -pos).all()         # sign-magnitude


def test_e4m3_encode_is_nearest_with_ties_to_even():
    rng = np.random.default_rng(1)
    finite = mla.e4m3_values()[:0x7F]
    x = np.concatenate([rng.uniform(-460, 460, 4000), rng.normal(0, 1, 4000), rng.normal(0, 0.01, 2000),
                        rng.uniform(-2.0 ** -6, 2.0 ** -6, 2000)])
    codes = mla.e4m3_encode(x)
    got = mla.e4m3_decode(codes)
    mag = np.minimum(np.abs(x), 448.0)
    best = np.min(np.abs(finite[None, :] - mag[:, None]), axis=1)
    assert np.array_equal(np.abs(np.abs(got) - mag), best)
    assert np.array_equal(np.signbit(got), np.signbit(x))
    # exact midpoints go to the code with an even mantissa
    assert mla.e4m3_encode(1.0625) == 0x38      # between 1.0 (0x38) and 1.125 (0x39)
    assert mla.e4m3_encode(1.1875) == 0x3A      # between 1.125 (0x39) and 1.25 (0x3a)
    assert mla.e4m3_encode(2.0 ** -10) == 0x00  # half the smallest subnormal
    assert mla.e4m3_encode(3 * 2.0 ** -10) == 0x02
    assert mla.e4m3_encode(432.0) == 0x7E       # between 416 (0x7d) and 448 (0x7e)


def test_e4m3_saturation_sign_and_round_trip():
    assert mla.e4m3_encode(1e9) == 0x7E and mla.e4m3_encode(-1e9) == 0xFE
    assert mla.e4m3_encode(449.0) == 0x7E
    assert mla.e4m3_encode(-0.0) == 0x80 and mla.e4m3_encode(0.0) == 0x00
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = mla.e4m3_encode(mla.e4m3_decode(codes))
    assert np.array_equal(back, codes)


# ------------------------------------------------------------- quantisation
def test_quantize_latent_scales_and_extremes():
    rng = np.random.default_rng(2)
    lat = rng.normal(0, 3, (40, 512)).astype(np.float32)
    lat[5, 128:256] = 0.0                       # an all-zero group
    lat[6, 127] = 1000.0                        # the last value of group 0
    lat[7, 128] = -1000.0                       # the first value of group 1
    codes, scales = mla.quantize_latent(lat)
    assert codes.shape == (40, 512) and codes.dtype == np.uint8 and scales.shape == (40, 4)
    amax = np.abs(lat.reshape(40, 4, 128)).max(axis=2)
    want = np.where(amax > 0, amax / np.float32(448), np.float32(1)).astype(np.float32)
    assert np.array_equal(scales, want)
    assert scales[5, 1] == 1.0 and (codes[5, 128:256] == 0).all()
    assert codes[6, 127] == 0x7E and scales[6, 0] == np.float32(1000.0) / np.float32(448)
    assert codes[7, 128] == 0xFE and scales[7, 0] < 100
    # every group's largest magnitude hits the top code
    g = codes.reshape(40, 4, 128)
    top = np.take_along_axis(g, np.abs(lat.reshape(40, 4, 128)).argmax(axis=2)[:, :, None], 2)[..., 0]
    assert ((top & 0x7F) == 0x7E)[amax > 0].all()


def test_quantize_error_bound_and_group_independence():
    rng = np.random.default_rng(3)
    lat = (rng.normal(0, 1, (64, 512)) * rng.uniform(0.01, 50, (64, 1))).astype(np.float32)
    codes, scales = mla.quantize_latent(lat)
    deq = mla.dequantize_latent(codes, scales)
    sc = np.repeat(scales.astype(np.float64), 128, axis=1)
    # three mantissa bits: half an ulp is 2^-4 relative for normals, 2^-10 * scale below 2^-6 * scale
    bound = np.maximum(np.abs(lat) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(deq - lat) <= bound).all()
    lat2 = lat.copy()
    lat2[:, 300] *= 100                          # group 2 only
    c2, s2 = mla.quantize_latent(lat2)
    assert np.array_equal(c2[:, :256], codes[:, :256]) and np.array_equal(c2[:, 384:], codes[:, 384:])
    assert np.array_equal(s2[:, [0, 1, 3]], scales[:, [0, 1, 3]])


def test_representable_latents_survive_fp8_exactly():
    rng = np.random.default_rng(4)
    vals = mla.e4m3_values()[:0x7F]
    lat = rng.choice(np.concatenate([vals, -vals]), (8, 512)).astype(np.float32)
    lat[:, ::128] = 448.0                        # amax 448 per group -> scale exactly 1
    bits = f32_to_bf16_bits(lat)
    rope = f32_to_bf16_bits(rng.normal(0, 1, (8, 64)))
    assert np.array_equal(mla.records(bits, rope, "fp8"), mla.records(bits, rope, "bf16"))


def test_fp8_records_keep_rope_bits():
    rng = np.random.default_rng(5)
    lat = f32_to_bf16_bits(rng.normal(0, 1, (10, 512)))
    rope = f32_to_bf16_bits(rng.normal(0, 1, (10, 64)))
    r8 = mla.records(lat, rope, "fp8")
    assert r8.shape == (10, 576)
    assert np.array_equal(r8[:, 512:], orc.bf16_bits_to_f64(rope))
    with pytest.raises(ValueError):
        mla.records(lat, rope, "fp4")


def test_per_token_bytes_match_the_deployment_notes():
    bf16_bytes = mla.RECORD * 2
    fp8_bytes = mla.LATENT * 1 + (mla.LATENT // mla.GROUP) * 4 + mla.ROPE * 2
    assert bf16_bytes == 1152 and fp8_bytes == 656
    assert round(bf16_bytes / fp8_bytes, 3) == 1.756


# ----------------------------------------------------------- absorbed decode
def test_absorbed_decode_equals_expanded_attention():
    rng = np.random.default_rng(6)
    heads, L, dn, dr = 4, 37, 128, 64
    lat = rng.normal(0, 1, (L, 512))
    rope = rng.normal(0, 1, (L, 64))
    w_uk = rng.normal(0, 512 ** -0.5, (heads, dn, 512))
    w_uv = rng.normal(0, 512 ** -0.5, (heads, dn, 512))
    q_nope = rng.normal(0, 1, (heads, dn))
    q_rope = rng.normal(0, 1, (heads, dr))
    scale = 1 / math.sqrt(dn + dr)
    # expanded: one key/value head per query head
    k = np.concatenate([np.einsum("hdc,lc->lhd", w_uk, lat), np.broadcast_to(rope[:, None, :], (L, heads, dr))], 2)
    v = np.einsum("hdc,lc->lhd", w_uv, lat)
    q = np.concatenate([q_nope, q_rope], 1)[None]
    ref_out, ref_lse = orc.attend_rows(q, np.ascontiguousarray(k), np.ascontiguousarray(v), L - 1, scale,
                                       np.zeros(heads, np.int64), np.arange(heads, dtype=np.int32))
    # absorbed: latent-space query, one shared record per token
    q_abs = np.concatenate([np.einsum("hdc,hd->hc", w_uk, q_nope), q_rope], 1)
    out_lat, lse = mla.decode(q_abs, np.concatenate([lat, rope], 1), scale)
    out = np.einsum("hdc,hc->hd", w_uv, out_lat)
    assert np.allclose(out, ref_out, rtol=1e-10, atol=1e-12)
    assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_decode_special_cases():
    rng = np.random.default_rng(7)
    recs = rng.normal(0, 1, (50, 576))
    q = f32_to_bf16_bits(rng.normal(0, 1, (16, 576)))
    out, lse = mla.decode(q, recs[:1], 0.1)
    assert np.array_equal(out, np.broadcast_to(recs[0, :512], (16, 512)))
    assert np.allclose(lse, 0.1 * orc.bf16_bits_to_f64(q) @ recs[0], rtol=1e-13, atol=1e-13)
    out, lse = mla.decode(np.zeros((16, 576)), recs, 0.3)
    assert np.allclose(out, recs[:, :512].mean(axis=0), rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, math.log(50), rtol=1e-13)
    # the output reads only the latent part: changing rotary values of equal-score records moves nothing
    q0 = np.zeros((16, 576))
    recs2 = recs.copy()
    recs2[:, 512:] = rng.normal(0, 1, (50, 64))
    assert np.allclose(mla.decode(q0, recs2, 0.3)[0], out, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------- absorbed prefill
def test_prefill_zero_query_averages_the_visible_records():
    rng = np.random.default_rng(8)
    past, c, heads = 45, 7, 16
    recs = rng.normal(0, 1, (past + c, 576))
    out, lse = mla.prefill(np.zeros((c, heads, 576)), recs, past, 0.2)
    for t in range(c):
        p = past + t
        for h in (0, 9, 15):
            i = t * heads + h
            assert np.allclose(out[i], recs[: p + 1, :512].mean(axis=0), rtol=1e-12, atol=1e-13)
            assert math.isclose(lse[i], math.log(p + 1), rel_tol=1e-13)


def test_prefill_first_position_and_causality():
    rng = np.random.default_rng(9)
    c, heads = 9, 32
    recs = rng.normal(0, 1, (c, 576))
    q = f32_to_bf16_bits(rng.normal(0, 1, (c, heads, 576)))
    out, lse = mla.prefill(q, recs, 0, 0.07)
    # position 0 sees record 0 alone
    assert np.array_equal(out[:heads], np.broadcast_to(recs[0, :512], (heads, 512)))
    assert np.allclose(lse[:heads], 0.07 * orc.bf16_bits_to_f64(q[0]) @ recs[0], rtol=1e-13, atol=1e-13)
    # records after a row's position do not move it: perturb record 5 onwards
    recs2 = recs.copy()
    recs2[5:] = rng.normal(0, 3, (c - 5, 576))
    out2, lse2 = mla.prefill(q, recs2, 0, 0.07)
    assert np.array_equal(out2[: 5 * heads], out[: 5 * heads]) and np.array_equal(lse2[: 5 * heads], lse[: 5 * heads])
    assert not np.allclose(out2[5 * heads:], out[5 * heads:])
    # records beyond the chunk are never read
    more = np.concatenate([recs, np.full((4, 576), np.nan)])
    out3, _ = mla.prefill(q, more, 0, 0.07)
    assert np.array_equal(out3, out)


def test_prefill_chunk_equals_expanded_attention():
    rng = np.random.default_rng(10)
    heads, past, c, dn, dr = 4, 29, 6, 128, 64
    L = past + c
    lat = rng.normal(0, 1, (L, 512))
    rope = rng.normal(0, 1, (L, 64))
    w_uk = rng.normal(0, 512 ** -0.5, (heads, dn, 512))
    w_uv = rng.normal(0, 512 ** -0.5, (heads, dn, 512))
    q_nope = rng.normal(0, 1, (c, heads, dn))
    q_rope = rng.normal(0, 1, (c, heads, dr))
    scale = 1 / math.sqrt(dn + dr)
    k = np.concatenate([np.einsum("hdc,lc->lhd", w_uk, lat), np.broadcast_to(rope[:, None, :], (L, heads, dr))], 2)
    v = np.einsum("hdc,lc->lhd", w_uv, lat)
    tok = np.repeat(np.arange(c, dtype=np.int64), heads)
    head = np.tile(np.arange(heads, dtype=np.int32), c)
    ref_out, ref_lse = orc.attend_rows(np.concatenate([q_nope, q_rope], 2), np.ascontiguousarray(k),
                                       np.ascontiguousarray(v), past, scale, tok, head)
    q_abs = np.concatenate([np.einsum("hdc,thd->thc", w_uk, q_nope), q_rope], 2)
    out_lat, lse = mla.prefill(q_abs, np.concatenate([lat, rope], 1), past, scale)
    out = np.stack([w_uv[h] @ out_lat[i] for i, h in enumerate(head)])
    assert np.allclose(out, ref_out, rtol=1e-10, atol=1e-12)
    assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_fp8_staged_records_round_code_times_scale_once_to_bf16():
    rng = np.random.default_rng(11)
    lat = rng.normal(0, 1, (40, 512)).astype(np.float32)
    lat[0, :128] = np.float32(448.0) * np.linspace(-1, 1, 128, dtype=np.float32)   # amax 448: scale 1
    lat[1, 128:256] = np.float32(448.0 * 2.0 ** -5) * np.sign(np.linspace(-1, 1, 128, dtype=np.float32))  # 2^-5
    lat_bits, rope_bits = f32_to_bf16_bits(lat), f32_to_bf16_bits(rng.normal(0, 1, (40, 64)))
    staged = mla.fp8_staged_records(lat_bits, rope_bits)
    exact = mla.records(lat_bits, rope_bits, "fp8")
    # representable in bf16: the low 16 bits of the fp32 pattern are zero
    assert not np.any(staged.astype(np.float32).view(np.uint32) & 0xFFFF)
    # within the bf16 rounding bound of the exact record; rotary parts untouched
    assert np.all(np.abs(staged - exact) <= 2.0 ** -8 * np.abs(exact) * (1 + 2.0 ** -20))
    assert np.array_equal(staged[:, 512:], exact[:, 512:])
    # power-of-two scales: code x scale is exact in bf16 (a 4-bit significand)
    assert np.array_equal(staged[0, :128], exact[0, :128]) and np.array_equal(staged[1, 128:256], exact[1, 128:256])
    # rounding is to nearest with ties to even: 1 + 2^-8 (a tie between 1 and 1 + 2^-7) goes to 1
    assert mla.f32_to_bf16_rne(np.float32(1 + 2.0 ** -8)) == 1.0
    assert mla.f32_to_bf16_rne(np.float32(1 + 3 * 2.0 ** -8)) == 1 + 2 * 2.0 ** -7
    assert mla.f32_to_bf16_rne(np.float32(1 + 2.0 ** -8 + 2.0 ** -20)) == 1 + 2.0 ** -7
