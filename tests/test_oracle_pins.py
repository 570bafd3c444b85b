"""Pins for the fp64 CPU oracle (CPU only).

The oracle is the plain definition of chunked-prefill causal attention (VPP
technical review, English edition, §2.2 Eq. (1) and its causal rule; §2.3 for
the chunk offset).  These tests tie it to things other than itself:

* hand-derived rational values (``tests/golden/rational_tiny.json``);
* closed forms: zero queries give the prefix mean of V, constant V gives that
  constant, a dominant key selects its value, the first row copies v_0;
* invariants: chunk concatenation equals one full causal pass (also for an
  uneven last chunk), rows ignore K/V beyond their position, a common shift
  of every key leaves the output unchanged, GQA equals MHA with replicated
  KV heads, an LSE merge over any key partition equals the single pass;
* a library routine on the same inputs: torch's ``scaled_dot_product_attention``
  and ``logsumexp`` in fp64 on the CPU with an explicit position mask;
* a pure-Python brute force with exactly rounded sums on tiny inputs.

Each pin is a function of an ``attend`` callable, so the same pins are run
against planted mistakes (``test_pins_catch_planted_mistakes``): every
mutant must fail at least one pin.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


# ---------------------------------------------------------------- helpers --

def c_attend(q, k, v, past_len, scale):
    """The oracle under test: out [c, Hq, dv], lse [Hq, c]."""
    return oracle.chunk_attention(np.asarray(q, np.float32), np.asarray(k, np.float32),
                                  np.asarray(v, np.float32), past_len, scale)


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def sdpa_reference(q, k, v, past_len, scale):
    """torch fp64 SDPA + logsumexp with an explicit absolute-position mask."""
    q = torch.from_numpy(np.asarray(q, np.float64))
    k = torch.from_numpy(np.asarray(k, np.float64))
    v = torch.from_numpy(np.asarray(v, np.float64))
    c, hq, _ = q.shape
    L, hkv, _ = k.shape
    g = hq // hkv
    kk = k.repeat_interleave(g, dim=1).permute(1, 0, 2)    # [Hq, L, d]
    vv = v.repeat_interleave(g, dim=1).permute(1, 0, 2)
    qq = q.permute(1, 0, 2)                                # [Hq, c, d]
    pos = past_len + torch.arange(c)[:, None]
    mask = torch.arange(L)[None, :] <= pos                 # [c, L]
    out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)
    logits = (qq @ kk.transpose(1, 2)) * scale
    lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)
    return out.permute(1, 0, 2).numpy(), lse.numpy()


# ------------------------------------------------------------------- pins --

def pin_golden(attend):
    with open(os.path.join(GOLDEN, "rational_tiny.json")) as f:
        g = json.load(f)
    out, lse = attend(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), g["past_len"], math.log(2.0))
    want = np.array([[[float(Fraction(x)) for x in row] for row in tok] for tok in g["out"]])
    want_lse = np.array([[math.log(float(s.split()[1])) for s in h] for h in g["lse"]])
    assert np.allclose(out, want, rtol=0, atol=1e-12), (out, want)
    assert np.allclose(lse, want_lse, rtol=0, atol=1e-12), (lse, want_lse)


def pin_zero_queries_give_prefix_mean(attend):
    k, v = rand((13, 2, 4), 1), rand((13, 2, 3), 2)
    q = np.zeros((5, 4, 4), np.float32)
    past = 8
    out, lse = attend(q, k, v, past, 0.5)
    for i in range(5):
        for h in range(4):
            want = v[: past + i + 1, h // 2].astype(np.float64).mean(axis=0)
            assert np.allclose(out[i, h], want, atol=TOL)
            assert abs(lse[h, i] - math.log(past + i + 1)) < TOL


def pin_constant_values(attend):
    q, k = rand((6, 2, 8), 3), rand((10, 1, 8), 4)
    u = np.array([0.25, -1.5, 3.0], np.float32)
    v = np.broadcast_to(u, (10, 1, 3)).copy()
    out, _ = attend(q, k, v, 4, 0.3)
    assert np.allclose(out, np.broadcast_to(u, out.shape), atol=TOL)


def pin_dominant_key(attend):
    q = rand((1, 1, 4), 5)
    k = rand((6, 1, 4), 6) * 0.01
    k[3, 0] = 50.0 * q[0, 0]
    v = rand((6, 1, 2), 7)
    out, _ = attend(q, k, v, 5, 1.0)
    assert np.allclose(out[0, 0], v[3, 0], atol=1e-9)


def pin_first_row_copies_v0(attend):
    q, k, v = rand((3, 2, 4), 8), rand((3, 1, 4), 9), rand((3, 1, 5), 10)
    out, lse = attend(q, k, v, 0, 0.7)
    for h in range(2):
        assert np.array_equal(out[0, h], v[0, 0].astype(np.float64))
        assert abs(lse[h, 0] - 0.7 * float(np.dot(q[0, h].astype(np.float64), k[0, 0].astype(np.float64)))) < TOL


def pin_chunks_equal_full_pass(attend):
    L, hq, hkv, d, dv = 23, 4, 2, 5, 3
    q, k, v = rand((L, hq, d), 11), rand((L, hkv, d), 12), rand((L, hkv, dv), 13)
    full, full_lse = attend(q, k, v, 0, 0.4)
    for bounds in ([0, 8, 16, 23], [0, 10, 20, 23], [0, 1, 2, 23]):   # even and uneven last chunk
        for a, b in zip(bounds[:-1], bounds[1:]):
            out, lse = attend(q[a:b], k[:b], v[:b], a, 0.4)
            assert np.allclose(out, full[a:b], atol=TOL)
            assert np.allclose(lse, full_lse[:, a:b], atol=TOL)


def pin_future_keys_ignored(attend):
    q, k, v = rand((4, 2, 6), 14), rand((12, 2, 6), 15), rand((12, 2, 4), 16)
    past = 5
    base, base_lse = attend(q, k, v, past, 0.6)
    for i in range(4):
        k2, v2 = k.copy(), v.copy()
        pos = past + i
        k2[pos + 1:] = rand(k2[pos + 1:].shape, 100 + i) * 7.0
        v2[pos + 1:] = rand(v2[pos + 1:].shape, 200 + i) * 7.0
        out, lse = attend(q, k2, v2, past, 0.6)
        assert np.array_equal(out[: i + 1], base[: i + 1])
        assert np.array_equal(lse[:, : i + 1], base_lse[:, : i + 1])


def pin_key_shift_invariance(attend):
    q, k, v = rand((5, 2, 4), 17), rand((9, 1, 4), 18), rand((9, 1, 3), 19)
    a = np.array([0.5, -0.25, 1.0, 0.125], np.float32)
    base, _ = attend(q, k, v, 4, 0.5)
    out, _ = attend(q, (k + a).astype(np.float32), v, 4, 0.5)
    # k + a is rounded to float32 before the oracle sees it, hence 1e-6 rather than 1e-12
    assert np.allclose(out, base, atol=1e-6)


def pin_gqa_equals_replicated_mha(attend):
    q, k, v = rand((6, 6, 4), 20), rand((10, 2, 4), 21), rand((10, 2, 3), 22)
    g, _ = attend(q, k, v, 4, 0.5)
    m, _ = attend(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), 4, 0.5)
    assert np.array_equal(g, m)


def pin_library_sdpa(attend):
    for seed, (c, past, hq, hkv, d, dv) in enumerate([(7, 0, 2, 2, 8, 8), (9, 11, 4, 1, 6, 5), (16, 3, 8, 2, 12, 4)]):
        L = past + c
        q, k, v = rand((c, hq, d), 30 + seed), rand((L, hkv, d), 40 + seed), rand((L, hkv, dv), 50 + seed)
        out, lse = attend(q, k, v, past, 1.0 / math.sqrt(d))
        ref, ref_lse = sdpa_reference(q, k, v, past, 1.0 / math.sqrt(d))
        assert np.allclose(out, ref, atol=1e-12), np.abs(out - ref).max()
        assert np.allclose(lse, ref_lse, atol=1e-12)


def pin_brute_force(attend):
    for seed, (c, past, hq, hkv, d, dv) in enumerate([(3, 0, 1, 1, 1, 1), (4, 5, 2, 1, 2, 3), (6, 2, 4, 2, 8, 2)]):
        L = past + c
        q, k, v = rand((c, hq, d), 60 + seed), rand((L, hkv, d), 70 + seed), rand((L, hkv, dv), 80 + seed)
        out, lse = attend(q, k, v, past, 0.9)
        bout, blse = brute.attend(q.tolist(), k.tolist(), v.tolist(), past, 0.9, hq // hkv)
        assert np.allclose(out, np.array(bout), atol=1e-12)
        assert np.allclose(lse, np.array(blse), atol=1e-12)


PINS = [pin_golden, pin_zero_queries_give_prefix_mean, pin_constant_values, pin_dominant_key,
        pin_first_row_copies_v0, pin_chunks_equal_full_pass, pin_future_keys_ignored,
        pin_key_shift_invariance, pin_gqa_equals_replicated_mha, pin_library_sdpa, pin_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(c_attend)


def test_oracle_bf16_inputs_widen_exactly():
    """bf16 bit patterns and their float32 values give bit-identical results."""
    q = torch.from_numpy(rand((5, 2, 8), 90)).to(torch.bfloat16)
    k = torch.from_numpy(rand((9, 1, 8), 91)).to(torch.bfloat16)
    v = torch.from_numpy(rand((9, 1, 4), 92)).to(torch.bfloat16)
    bits = [t.view(torch.int16).numpy().view(np.uint16) for t in (q, k, v)]
    out_b, lse_b = oracle.chunk_attention(*bits, 4, 0.35)
    out_f, lse_f = oracle.chunk_attention(*[t.float().numpy() for t in (q, k, v)], 4, 0.35)
    assert np.array_equal(out_b, out_f) and np.array_equal(lse_b, lse_f)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits[0]), q.double().numpy())


def test_oracle_sampled_rows_match_full():
    q, k, v = rand((12, 4, 8), 93), rand((20, 2, 8), 94), rand((20, 2, 6), 95)
    full, full_lse = oracle.chunk_attention(q, k, v, 8, 0.5)
    tok = np.array([0, 11, 5, 5, 7]); head = np.array([0, 3, 1, 2, 0], np.int32)
    out, lse = oracle.attend_rows(q, k, v, 8, 0.5, tok, head)
    assert np.array_equal(out, full[tok, head])
    assert np.array_equal(lse, full_lse[head, tok])


def test_oracle_merge_over_any_partition_equals_single_pass():
    """LSE merge of key-range partials (the split-KV merge) equals one pass."""
    c, past, hq, hkv, d, dv = 6, 30, 4, 2, 8, 5
    q, k, v = rand((c, hq, d), 96), rand((past + c, hkv, d), 97), rand((past + c, hkv, dv), 98)
    full, full_lse = oracle.chunk_attention(q, k, v, past, 0.4)
    tok = np.repeat(np.arange(c), hq); head = np.tile(np.arange(hq, dtype=np.int32), c)
    for cuts in ([0, 36], [0, 17, 36], [0, 1, 2, 33, 34, 36], [0, 33, 35, 36]):
        parts = [oracle.attend_rows(q, k, v, past, 0.4, tok, head, key_range=(a, b))
                 for a, b in zip(cuts[:-1], cuts[1:])]
        o, lse = oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        assert np.allclose(o.reshape(c, hq, dv), full, atol=1e-12)
        assert np.allclose(lse.reshape(c, hq).T, full_lse, atol=1e-12)
    # a key range that a row cannot see yields weight zero (lse = -inf)
    o, lse = oracle.attend_rows(q, k, v, past, 0.4, tok[:1], head[:1], key_range=(31, 36))
    assert lse[0] == -math.inf and np.all(o == 0)


def test_oracle_partial_range_matches_library():
    """A single key-range partial equals SDPA over that range (same mask logic)."""
    c, past, hq, hkv, d, dv = 5, 9, 2, 1, 4, 3
    q, k, v = rand((c, hq, d), 99), rand((past + c, hkv, d), 100), rand((past + c, hkv, dv), 101)
    lo, hi = 4, 12
    tok = np.repeat(np.arange(c), hq); head = np.tile(np.arange(hq, dtype=np.int32), c)
    o, lse = oracle.attend_rows(q, k, v, past, 0.5, tok, head, key_range=(lo, hi))
    qq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)
    kk = torch.from_numpy(k.astype(np.float64)).repeat_interleave(hq, 1).permute(1, 0, 2)
    vv = torch.from_numpy(v.astype(np.float64)).repeat_interleave(hq, 1).permute(1, 0, 2)
    j = torch.arange(past + c)[None, :]
    mask = (j <= past + torch.arange(c)[:, None]) & (j >= lo) & (j < hi)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=0.5)
    assert np.allclose(o.reshape(c, hq, dv), ref.permute(1, 0, 2).numpy(), atol=1e-12)
    ref_lse = torch.logsumexp(((qq @ kk.transpose(1, 2)) * 0.5).masked_fill(~mask, -math.inf), -1)
    assert np.allclose(lse.reshape(c, hq).T, ref_lse.numpy(), atol=1e-12)


def test_oracle_rejects_bad_rows():
    q, k, v = rand((4, 2, 4), 1), rand((6, 1, 4), 2), rand((6, 1, 2), 3)
    with pytest.raises(ValueError):
        oracle.attend_rows(q, k, v, 3, 0.5, np.array([3]), np.array([0], np.int32))   # position 6 >= kv_len
    with pytest.raises(ValueError):
        oracle.attend_rows(q, k, v, 0, 0.5, np.array([0]), np.array([2], np.int32))   # head out of range


# ------------------------------------------------------- planted mistakes --

def _numpy_attend(q, k, v, past_len, scale, mutation=None):
    """A test-only numpy restatement used as the base for planted mistakes."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    c, hq, d = q.shape
    L, hkv, _ = k.shape
    grp = hq // hkv
    if mutation == "transposed_q":
        q = q.reshape(hq, c, d).transpose(1, 0, 2)
    out = np.zeros((c, hq, v.shape[2])); lse = np.zeros((hq, c))
    for i in range(c):
        pos = i if mutation == "ignore_past" else past_len + i
        for h in range(hq):
            g = h % hkv if mutation == "gqa_modulo" else h // grp
            hi = L if mutation == "no_mask" else pos + 1 + (1 if mutation == "mask_off_by_one" else 0)
            hi = min(hi, L)
            sc = 1.0 if mutation == "no_scale" else scale
            s = sc * (k[:hi, g] @ q[i, h])
            if mutation == "sign":
                s = -s
            m = s.max(); w = np.exp(s - m); l = w.sum()
            vg = 0 if mutation == "v_head0" else g
            o = w @ v[:hi, vg]
            out[i, h] = o if mutation == "no_normalise" else o / l
            lse[h, i] = m + (np.log2(l) if mutation == "lse_log2" else np.log(l))
    return out, lse


MUTATIONS = ["no_mask", "mask_off_by_one", "ignore_past", "gqa_modulo", "no_scale", "transposed_q",
             "sign", "no_normalise", "lse_log2", "v_head0"]


def test_numpy_restatement_passes_pins():
    for pin in PINS:
        pin(lambda q, k, v, p, s: _numpy_attend(q, k, v, p, s))


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_pins_catch_planted_mistakes(mutation):
    caught = []
    for pin in PINS:
        try:
            pin(lambda q, k, v, p, s: _numpy_attend(q, k, v, p, s, mutation))
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin detects the planted mistake {mutation!r}"
