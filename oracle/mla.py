"""TEST INFRASTRUCTURE ONLY — plain reference of MLA latent (absorbed) decode
over a latent KV cache, in bf16 or in an fp8 latent format.

Only ``tests/`` may import this module; the library never does.

What the pages fix ("02 · 并行策略与 PP 切分 — GLM5.3 CyberSec W4A16"
deployment notes, §1 and §4): an MLA attention layer caches one latent
record per token that every query head shares (the KV is replicated across
tensor-parallel ranks, not split by head); that record takes 1152 B in bf16
and 656 B in the ``fp8_ds_mla`` format, a 1.756x ratio.  The VPP review's
models (DeepSeek-V3.1, GLM-5.x) use MLA attention (§6.1).

Readings (also in the design notes):

* Record = a 512-value latent plus a 64-value rotary part: 576 bf16 values
  (1152 B).  In fp8: the latent as 512 e4m3 codes with one fp32 scale per
  128 values, and the rotary part kept in bf16: 512 + 4 * 4 + 64 * 2 = 656 B.
  fp8 is OCP e4m3 ("e4m3fn": bias 7, subnormals, no infinities, largest
  normal 448).  A group's scale is amax / 448 in fp32 (1 when the group is all
  zero), and a value's code is its fp32 quotient by the scale, clamped to
  +-448 and rounded to the nearest code, ties to the even code.
* Absorbed decode: a query head carries 576 values (its latent-space
  projection of the no-rope part, then the rotary part).  Keys are the
  records, values are the 512-value latents of the same records, and the
  output stays in latent space (512 values per head).  With dequantized
  records this is plain attention with d_qk = 576, d_v = 512 and one KV head
  shared by every query head — computed by the package's fp64 oracle.
* A decode query sits at position kv_len - 1 and sees all kv_len records.
* Absorbed prefill (VPP review §2.3, chunked prefill; §2.2 Eq. (1) for the
  causal rule): a chunk of c tokens at positions past_len .. past_len + c - 1
  of one sequence; every head of the token at position p sees records
  0 .. p.  The same plain attention, row by row.
* Prefill over an fp8 cache runs its matrix products in bf16: a record
  enters as bf16(fp32(code x scale)) (``fp8_staged_records``), one more
  relative rounding of at most 2^-8 per value than the exact fp8 record.
"""
from __future__ import annotations

import numpy as np

import oracle as _orc

LATENT, ROPE = 512, 64
RECORD = LATENT + ROPE
GROUP = 128
E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """Value of every byte code 0..255 (NaN for the two NaN codes)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_VALS = e4m3_values()
_POS = _VALS[:0x7F]            # codes 0x00 .. 0x7e: every finite non-negative value, increasing


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of each float (ties to the even code), saturating at +-448.
    The sign bit follows the float's sign bit (so -0.0 gives 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS, mag, side="left")           # first code whose value >= mag
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS[hi] - mag
    d_lo = mag - _POS[lo]
    take_hi = (d_hi == 0) | (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    return _VALS[np.asarray(codes, dtype=np.uint8)]


def quantize_latent(latent_f32) -> tuple[np.ndarray, np.ndarray]:
    """fp8_ds_mla latent: codes [n, 512] uint8 and scales [n, 4] float32 from fp32 latents."""
    lat = np.asarray(latent_f32, dtype=np.float32).reshape(-1, LATENT // GROUP, GROUP)
    amax = np.max(np.abs(lat), axis=2)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    quot = (lat / scale[:, :, None]).astype(np.float32)           # fp32 division, correctly rounded
    codes = e4m3_encode(np.clip(quot, -E4M3_MAX, E4M3_MAX))
    return codes.reshape(-1, LATENT), scale


def dequantize_latent(codes, scales) -> np.ndarray:
    """fp64 latents code * scale (exact: a 4-bit significand times an fp32 scale)."""
    v = e4m3_decode(codes).reshape(-1, LATENT // GROUP, GROUP)
    return (v * np.asarray(scales, dtype=np.float64)[:, :, None]).reshape(-1, LATENT)


def records(latent_bits, rope_bits, fmt: str) -> np.ndarray:
    """The fp64 key records [n, 576] the attention sees for a bf16 ('bf16') or fp8 ('fp8') cache,
    from bf16 bit patterns of the latents [n, 512] and rotary parts [n, 64]."""
    lat = _orc.bf16_bits_to_f64(latent_bits)
    rope = _orc.bf16_bits_to_f64(rope_bits)
    if fmt == "fp8":
        lat = dequantize_latent(*quantize_latent(lat.astype(np.float32)))
    elif fmt != "bf16":
        raise ValueError(fmt)
    return np.concatenate([lat, rope], axis=1)


def f32_to_bf16_rne(x) -> np.ndarray:
    """fp32 values rounded to bf16, nearest with ties to even, returned as fp64 (finite inputs)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def fp8_staged_records(latent_bits, rope_bits) -> np.ndarray:
    """The records chunked prefill over an fp8 cache computes with: each latent value is its e4m3 code times
    its group's fp32 scale, the product rounded to fp32 and then to bf16 (both nearest, ties to even); the
    rotary part is bf16 already.  fp64 [n, 576]."""
    lat = _orc.bf16_bits_to_f64(latent_bits).astype(np.float32)
    codes, scales = quantize_latent(lat)
    prod = e4m3_decode(codes).astype(np.float32).reshape(-1, LATENT // GROUP, GROUP) * scales[:, :, None]
    lat_b = f32_to_bf16_rne(prod.astype(np.float32)).reshape(-1, LATENT)
    return np.concatenate([lat_b, _orc.bf16_bits_to_f64(rope_bits)], axis=1)


def decode(q, recs, scale: float, threads: int | None = None):
    """Absorbed decode of one request: q [H, 576] (bf16 bit patterns as uint16, or fp64 values),
    records [L, 576] (fp64).  Returns out [H, 512] and lse [H] (natural log), fp64."""
    q = np.asarray(q)
    q = _orc.bf16_bits_to_f64(q) if q.dtype == np.uint16 else np.asarray(q, dtype=np.float64)
    q = np.ascontiguousarray(q).reshape(1, -1, RECORD)
    k = np.ascontiguousarray(recs, dtype=np.float64).reshape(-1, 1, RECORD)
    v = np.ascontiguousarray(k[:, :, :LATENT])
    heads = q.shape[1]
    out, lse = _orc.attend_rows(q, k, v, k.shape[0] - 1, scale, np.zeros(heads, np.int64),
                                np.arange(heads, dtype=np.int32), threads=threads)
    return out, lse


def prefill(q, recs, past_len: int, scale: float, tok=None, head=None, threads: int | None = None):
    """Absorbed prefill of one chunk: q [c, H, 576] (bf16 bit patterns as uint16, or fp64 values),
    records [>= past_len + c, 576] (fp64) of the sequence.  Row (tok[i], head[i]) sits at position
    past_len + tok[i] and sees records 0 .. past_len + tok[i].  Every row by default.
    Returns out [n, 512] and lse [n] (natural log), fp64."""
    q = np.asarray(q)
    q = _orc.bf16_bits_to_f64(q) if q.dtype == np.uint16 else np.asarray(q, dtype=np.float64)
    c, heads = q.shape[0], q.shape[1]
    q = np.ascontiguousarray(q).reshape(c, heads, RECORD)
    if tok is None:
        tok = np.repeat(np.arange(c, dtype=np.int64), heads)
        head = np.tile(np.arange(heads, dtype=np.int32), c)
    n_keys = past_len + c
    k = np.ascontiguousarray(np.asarray(recs, dtype=np.float64)[:n_keys]).reshape(n_keys, 1, RECORD)
    v = np.ascontiguousarray(k[:, :, :LATENT])
    return _orc.attend_rows(q, k, v, past_len, scale, np.asarray(tok, dtype=np.int64),
                            np.asarray(head, dtype=np.int32), threads=threads)
