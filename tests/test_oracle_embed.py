"""Pins of the oracle's bfloat16 rounding and packed-embedding rows (CPU only).

orc_f64_to_bf16_bits is checked against a brute-force nearest-value search and
against torch's float32 -> bfloat16 conversion (round to nearest even) on
float32 inputs; orc_embed against the oracle's dequantised rows and that same
library conversion.  Source of the operation: deep-fold README, "Method"
(embeddings decode only the requested rows).
"""
import numpy as np
import pytest
import torch

import oracle


def _bf16_value(bits):
    return float(np.array([bits << 16], np.uint32).view(np.float32)[0])


def _nearest_bf16_brute(v):
    """Among bf16 patterns around v, the nearest to v (ties: even significand)."""
    f = np.float32(v)
    b0 = int(np.array([f], np.float32).view(np.uint32)[0] >> 16)
    best = None
    for b in range(max(b0 - 2, 0), min(b0 + 3, 0x7F80) + 1):
        if (b & 0x7F80) == 0x7F80 and b != 0x7F80:
            continue
        val = _bf16_value(b)
        d = abs(val - v)
        key = (d, b & 1)
        if best is None or key < best[0]:
            best = (key, b)
    return best[1]


def test_bf16_rounding_hand_values():
    assert oracle.f64_to_bf16_bits(1.0) == 0x3F80
    assert oracle.f64_to_bf16_bits(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even
    assert oracle.f64_to_bf16_bits(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even
    assert oracle.f64_to_bf16_bits(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # just past
    assert oracle.f64_to_bf16_bits(-0.0) == 0x8000
    assert oracle.f64_to_bf16_bits(float("nan")) == 0x7FC0
    assert oracle.f64_to_bf16_bits(float("-inf")) == 0xFF80
    assert oracle.f64_to_bf16_bits(2.0 ** -130) == 0x0008               # subnormal
    assert oracle.f64_to_bf16_bits(3.4e38) == 0x7F80                    # overflow


def test_bf16_rounding_brute_force():
    rng = np.random.default_rng(5)
    vals = rng.standard_normal(4000) * np.exp2(rng.integers(-60, 60, 4000))
    for v in vals:
        v = float(v)
        want = _nearest_bf16_brute(abs(v)) | (0x8000 if v < 0 else 0)
        assert oracle.f64_to_bf16_bits(v) == want, v


def test_bf16_rounding_matches_torch_on_float32():
    rng = np.random.default_rng(6)
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-100, 100, 20000))).astype(np.float32)
    # include exact ties: bf16 values plus half a bf16 ulp
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16) | 0x8000
    f = np.concatenate([f, ties.view(np.float32)])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16_bits(float(x)) for x in f], np.uint16)
    assert np.array_equal(got, want)


def _packed(N, K, seed, sigma=0.02):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * sigma).astype(np.float32)
    p, s, st = oracle.quantize_pack(W)
    assert st == 0
    return p, s


def test_embed_rows_match_dequant_and_library_rounding():
    p, s = _packed(40, 256, 7)
    ids = np.array([3, 0, 39, 3, 17], np.int64)
    out, st = oracle.embed(p, s, ids)
    assert st == 0 and out.shape == (5, 256)
    w32 = oracle.dequant_f32(p, s)[ids]          # fp32(L * s), one rounding
    w64 = oracle.dequant_f64(p, s)[ids]          # exact
    via_torch = torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # double rounding can only differ where the fp32 value sits on a bf16 tie
    tie = (w32.view(np.uint32) & 0xFFFF) == 0x8000
    assert np.array_equal(out[~tie], via_torch[~tie])
    for (i, k) in zip(*np.nonzero(tie)):
        assert out[i, k] == _nearest_bf16_brute(abs(w64[i, k])) | (0x8000 if w64[i, k] < 0 else 0)
    # repeated ids give identical rows; the zero level gives +0
    assert np.array_equal(out[0], out[3])
    codes = oracle.unpack_codes(p)[ids]
    assert np.all(out[codes == 7] == 0)


def test_embed_bad_ids_and_empty():
    p, s = _packed(8, 128, 8)
    out, st = oracle.embed(p, s, np.array([-1, 2, 8, 1 << 40], np.int64))
    assert st == oracle.EMBED_BAD_ID
    assert np.all(out[[0, 2, 3]] == 0) and np.any(out[1] != 0)
    out, st = oracle.embed(p, s, np.zeros(0, np.int64))
    assert out.shape == (0, 128) and st == 0


def test_embed_scale_is_exact_power_of_two_multiple():
    # one group, all codes 15 (level +1): the row is bf16(s) exactly
    p = np.full((1, 32), 0xFF, np.uint8)
    for sbits in (0x3C00, 0x2E66, 0x7BFF, 0x0001):
        s = np.array([[sbits]], np.uint16)
        out, _ = oracle.embed(p, s, np.array([0], np.int64))
        assert np.all(out == oracle.f64_to_bf16_bits(oracle.f16_bits_to_f64(sbits)))
