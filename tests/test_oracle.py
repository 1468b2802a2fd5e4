"""Pins for the CPU oracle: each check ties it to something other than itself
(library routines, published values, closed forms, brute force, invariants).

Inputs are seeded numpy draws; no value here comes from the HIP library.
"""
import os
import statistics

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_qlora():
    vals = []
    with open(os.path.join(GOLDEN, "qlora_nf4_levels.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            i, v = line.split()
            vals.append(float(v))
    assert len(vals) == 16
    return np.array(vals)


def _np_f16_bits(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def _f16_value(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


# ----------------------------------------------------------------- quantile
def test_normal_quantile_vs_library_routines():
    from scipy.special import ndtri
    nd = statistics.NormalDist()
    ps = np.concatenate([np.linspace(0.5, 0.99, 200), [1e-6, 1e-3, 0.02, 0.25, 0.9677083333333333,
                                                       0.999, 0.999999]])
    for p in ps:
        x = oracle.normal_quantile(p)
        ref1 = nd.inv_cdf(p) if p != 0.5 else 0.0
        ref2 = float(ndtri(p))
        tol = 1e-12 * max(1.0, abs(ref2))
        assert abs(x - ref1) <= tol, (p, x, ref1)
        assert abs(x - ref2) <= tol, (p, x, ref2)


# ----------------------------------------------------------------- codebook
def test_codebook_invariants():
    l64, l32 = oracle.codebook()
    assert l64.shape == (16,) and l32.shape == (16,)
    assert l64[0] == -1.0 and l64[15] == 1.0 and l64[7] == 0.0
    assert np.all(np.diff(l64) > 0)
    assert (l64 < 0).sum() == 7 and (l64 > 0).sum() == 8
    # stored table is the fp32 rounding (numpy's RNE conversion) of the fp64 levels
    assert np.array_equal(l32, l64.astype(np.float32))
    assert l32.view(np.uint32)[7] == 0  # +0, not -0


def test_codebook_vs_qlora_printed_table():
    l64, l32 = oracle.codebook()
    q = _load_qlora()
    assert np.max(np.abs(l64 - q)) < 1e-6
    assert np.max(np.abs(l32.astype(np.float64) - q)) < 1e-6


def test_codebook_gaps():
    # the widest gap (between the two lowest levels) bounds the quantization error
    l64, _ = oracle.codebook()
    gaps = np.diff(l64)
    assert np.argmax(gaps) == 0
    assert 0.3 < gaps.max() < 0.31


# ----------------------------------------------------------------- binary16
def test_f16_hand_values():
    assert oracle.f32_to_f16_bits(1.0) == 0x3C00
    assert oracle.f32_to_f16_bits(0.1) == 0x2E66
    assert oracle.f32_to_f16_bits(65504.0) == 0x7BFF
    assert oracle.f32_to_f16_bits(65519.0) == 0x7BFF
    assert oracle.f32_to_f16_bits(65520.0) == 0x7C00
    assert oracle.f32_to_f16_bits(2.0 ** -24) == 0x0001
    assert oracle.f32_to_f16_bits(2.0 ** -25) == 0x0000       # tie -> even (0)
    assert oracle.f32_to_f16_bits(1.5 * 2.0 ** -24) == 0x0002  # tie -> even (2)
    assert oracle.f32_to_f16_bits(-2.0) == 0xC000
    assert oracle.f32_to_f16_bits(0.0) == 0x0000


def test_f16_conversion_vs_numpy():
    rng = np.random.default_rng(11)
    # log-uniform magnitudes across subnormal .. overflow, both signs
    mags = np.exp(rng.uniform(np.log(2.0 ** -27), np.log(7.0e4), 20000)).astype(np.float32)
    vals = np.concatenate([mags, -mags[:2000]])
    # exact midpoints between neighbouring fp16 values (ties): representable in fp32
    h = rng.integers(0, 0x7BFF, 3000).astype(np.uint16)
    lo = _f16_value(h)
    hi = _f16_value(h + 1)
    mids = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (lo + hi) / 2)
    vals = np.concatenate([vals, mids])
    ref = _np_f16_bits(vals)
    got = np.array([oracle.f32_to_f16_bits(v) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


def test_f16_and_bf16_decode_every_pattern():
    for b in range(0, 65536, 7):
        ref = float(np.uint16(b).view(np.float16))
        got = oracle.f16_bits_to_f64(b)
        if np.isnan(ref):
            assert np.isnan(got)
        else:
            assert got == ref, hex(b)
        refb = float(np.array([b << 16], np.uint32).view(np.float32)[0])
        gotb = oracle.bf16_bits_to_f64(b)
        if np.isnan(refb):
            assert np.isnan(gotb)
        else:
            assert gotb == refb, hex(b)


# ----------------------------------------------------------------- quantize
def _brute_force(W):
    """Nearest level by exhaustive search over all 16 codes, ties -> lower code."""
    _, l32 = oracle.codebook()
    N, K = W.shape
    scale_bits = np.zeros((N, K // 64), np.uint16)
    codes = np.zeros((N, K), np.uint8)
    for n in range(N):
        for g in range(K // 64):
            w = W[n, g * 64:(g + 1) * 64].astype(np.float64)
            sb = _np_f16_bits(np.float32(np.max(np.abs(W[n, g * 64:(g + 1) * 64]))))
            scale_bits[n, g] = sb
            s = float(_f16_value(sb))
            for k in range(64):
                if s == 0.0:
                    codes[n, g * 64 + k] = 7
                    continue
                d = np.abs(w[k] - l32.astype(np.float64) * s)
                codes[n, g * 64 + k] = int(np.flatnonzero(d == d.min())[0])
    return codes, scale_bits


@pytest.mark.parametrize("seed,sigma", [(1, 0.02), (2, 1.0), (3, 0.015), (4, 3e-5), (5, 900.0)])
def test_quantize_brute_force_2x64(seed, sigma):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((2, 64)) * sigma).astype(np.float32)
    codes, scales, st = oracle.quantize(W)
    bc, bs = _brute_force(W)
    assert st == 0
    assert np.array_equal(scales, bs)
    assert np.array_equal(codes, bc)


def test_quantize_brute_force_wider_shapes():
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((3, 256)) * 0.02).astype(np.float32)
    W[1, 64:128] *= 1e-3
    W[2, :64] = rng.uniform(-1, 1, 64).astype(np.float32)
    codes, scales, st = oracle.quantize(W)
    bc, bs = _brute_force(W)
    assert st == 0 and np.array_equal(scales, bs) and np.array_equal(codes, bc)


def test_quantize_adversarial_boundaries():
    """Weights on and one ulp around every decision boundary, scale fixed at 1."""
    _, l32 = oracle.codebook()
    mids = (l32[:-1].astype(np.float64) + l32[1:].astype(np.float64)) / 2
    vals = []
    for m in mids:
        f = np.float32(m)
        vals += [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))]
    vals += [np.float32(0.0), np.float32(-0.0), np.float32(1.0), np.float32(-1.0)]
    vals = np.array(vals, np.float32)
    pad = (-len(vals)) % 64
    row = np.concatenate([vals, np.zeros(pad, np.float32)])
    row[-1] = 1.0  # absmax 1 -> scale exactly 1.0
    W = row.reshape(1, -1)
    codes, scales, st = oracle.quantize(W)
    bc, bs = _brute_force(W)
    assert st == 0
    assert np.all(scales == 0x3C00)
    assert np.array_equal(codes, bc)
    # boundaries that are exactly representable are ties and go to the lower code
    for i, m in enumerate(mids):
        if np.float64(np.float32(m)) == m:
            W1 = np.zeros((1, 64), np.float32)
            W1[0, 0] = np.float32(m)
            W1[0, 1] = 1.0
            c1, _, _ = oracle.quantize(W1)
            assert c1[0, 0] == i, (i, m)


def test_quantize_round_trip_every_code():
    """quantize(L[c]*s) == c for every code, over many scales."""
    _, l32 = oracle.codebook()
    rng = np.random.default_rng(21)
    sbits = rng.integers(0x0400, 0x7800, 2000).astype(np.uint16)  # normal fp16 scales
    for sb in sbits:
        s = float(_f16_value(sb))
        row = np.zeros(64, np.float32)
        row[:16] = (l32.astype(np.float64) * s).astype(np.float32)
        row[16:32] = row[:16]
        row[32:] = np.float32(0.0)
        W = row.reshape(1, 64)
        codes, scales, st = oracle.quantize(W)
        assert st == 0 and scales[0, 0] == sb
        assert np.array_equal(codes[0, :16], np.arange(16))
        assert np.array_equal(codes[0, 16:32], np.arange(16))
        assert np.all(codes[0, 32:] == 7)


def test_quantize_error_bound():
    l64, l32 = oracle.codebook()
    half_gap = np.max(np.diff(l32.astype(np.float64))) / 2
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    packed, scales, st = oracle.quantize_pack(W)
    Wt = oracle.dequant_f64(packed, scales)
    s = _f16_value(scales).repeat(64, axis=1)
    amax = np.abs(W.astype(np.float64)).reshape(16, 8, 64).max(axis=2).repeat(64, axis=1)
    bound = half_gap * s + np.maximum(amax - s, 0.0)
    assert np.all(np.abs(W - Wt) <= bound + 1e-300)


def test_quantize_scale_invariance():
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((4, 128)) * 0.5).astype(np.float32)
    c0, s0, _ = oracle.quantize(W)
    for e in (-6, -1, 1, 3):
        c1, s1, _ = oracle.quantize((W * np.float32(2.0 ** e)).astype(np.float32))
        assert np.array_equal(c0, c1)
        assert np.array_equal(_f16_value(s1), _f16_value(s0) * 2.0 ** e)


def test_quantize_zero_and_tiny_groups():
    W = np.zeros((1, 128), np.float32)
    W[0, 64:] = np.float32(2.0 ** -26)  # absmax below half the smallest subnormal
    codes, scales, st = oracle.quantize(W)
    assert st == 0 and np.all(scales == 0) and np.all(codes == 7)
    W[0, 0] = -0.0
    codes, scales, st = oracle.quantize(W)
    assert np.all(codes == 7)


def test_quantize_flags_nonfinite_and_overflow():
    W = np.full((2, 192), 0.5, np.float32)
    W[0, 3] = np.nan
    W[1, 70] = np.inf
    W[1, 130] = 70000.0
    codes, scales, st = oracle.quantize(W)
    assert st == (oracle.STATUS_NONFINITE | oracle.STATUS_SCALE_OVERFLOW)
    assert scales[0, 0] == 0 and np.all(codes[0, :64] == 7)
    assert scales[1, 1] == 0 and np.all(codes[1, 64:128] == 7)
    assert scales[1, 2] == 0 and np.all(codes[1, 128:] == 7)
    assert scales[0, 1] == 0x3800 and scales[1, 0] == 0x3800  # 0.5, untouched groups
    # absmax 65519 still fits (rounds to 65504)
    W2 = np.full((1, 64), 65519.0, np.float32)
    _, s2, st2 = oracle.quantize(W2)
    assert st2 == 0 and s2[0, 0] == 0x7BFF


# ----------------------------------------------------------------- packing
def _load_pack_vectors():
    rows = []
    with open(os.path.join(GOLDEN, "pack_hand_vector.txt")) as f:
        lines = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for a, b in zip(lines[0::2], lines[1::2]):
        assert a[0] == "codes" and b[0] == "bytes"
        rows.append(([int(v) for v in a[1:]], [int(v, 16) for v in b[1:]]))
    return rows


def test_pack_hand_vector():
    for codes, bytes_ in _load_pack_vectors():
        c = np.array(codes * 4, np.uint8).reshape(1, 64)
        p = oracle.pack(c)
        assert list(p[0, :8]) == bytes_
        assert np.array_equal(oracle.unpack_codes(p), c)


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 16, (5, 320)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_codes(oracle.pack(c)), c)


def test_payload_ratio_matches_readme():
    # deep-fold README, Method: code-and-scale payload about 3.76x smaller than BF16
    N, K = 4096, 4096
    packed_bytes = N * K // 2 + N * (K // 64) * 2
    assert packed_bytes == N * K * 17 // 32
    ratio = 2 * N * K / packed_bytes
    assert abs(ratio - 3.76) < 0.01


# ----------------------------------------------------------------- dequant
def test_dequant_special_codes_and_fp32_rounding():
    _, l32 = oracle.codebook()
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 16, (3, 128)).astype(np.uint8)
    codes[0, :3] = [0, 7, 15]
    scales = rng.integers(0x0001, 0x7BFF, (3, 2)).astype(np.uint16)
    packed = oracle.pack(codes)
    W64 = oracle.dequant_f64(packed, scales)
    W32 = oracle.dequant_f32(packed, scales)
    s = _f16_value(scales).repeat(64, axis=1)
    assert W64[0, 0] == -s[0, 0] and W64[0, 1] == 0.0 and W64[0, 2] == s[0, 2]
    # fp32 path == numpy's correctly rounded fp32 multiply of level and scale
    ref32 = l32[codes] * s.astype(np.float32)
    assert np.array_equal(W32.view(np.uint32), ref32.astype(np.float32).view(np.uint32))
    assert np.array_equal(W64, l32[codes].astype(np.float64) * s)


# ----------------------------------------------------------------- product
def _bf16_bits(x):
    """fp32 -> bf16 bits, round to nearest even (via torch's conversion)."""
    import torch
    t = torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("M,N,K", [(1, 2, 64), (3, 2, 64), (2, 5, 192), (4, 3, 320)])
def test_gemm_vs_numpy_matmul(M, N, K):
    _, l32 = oracle.codebook()
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    scales = _np_f16_bits(rng.uniform(0.001, 0.1, (N, K // 64)))
    X = _bf16_bits(rng.standard_normal((M, K)))
    Y, A = oracle.gemm(oracle.pack(codes), scales, X)
    Wt = l32[codes].astype(np.float64) * _f16_value(scales).repeat(64, axis=1)
    Xv = _bf16_value(X)
    ref = Xv @ Wt.T
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-15)
    assert np.allclose(A, np.abs(Xv) @ np.abs(Wt).T, rtol=1e-12, atol=1e-15)


def test_gemm_closed_forms():
    _, l32 = oracle.codebook()
    rng = np.random.default_rng(8)
    N, K = 4, 128
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    scales = _np_f16_bits(rng.uniform(0.01, 0.1, (N, K // 64)))
    packed = oracle.pack(codes)
    # x = 0 -> y = 0
    Y, A = oracle.gemm(packed, scales, np.zeros(K, np.uint16))
    assert np.all(Y == 0) and np.all(A == 0)
    # every code the zero level -> y = 0
    Y, _ = oracle.gemm(oracle.pack(np.full((N, K), 7, np.uint8)), scales,
                       _bf16_bits(rng.standard_normal(K)))
    assert np.all(Y == 0)
    # a constant code c in one group, x = 1 there and 0 elsewhere -> 64 * L[c] * s
    one = _bf16_bits(np.concatenate([np.ones(64), np.zeros(K - 64)]))
    for c in range(16):
        cc = np.full((1, K), c, np.uint8)
        Y, _ = oracle.gemm(oracle.pack(cc), scales[:1], one)
        assert Y[0, 0] == 64 * float(l32[c]) * float(_f16_value(scales[0, 0]))
    # x = e_k -> column k of the dequantized matrix
    W64 = oracle.dequant_f64(packed, scales)
    for k in (0, 1, 63, 64, 127):
        e = np.zeros(K, np.float32)
        e[k] = 1.0
        Y, _ = oracle.gemm(packed, scales, _bf16_bits(e))
        assert np.array_equal(Y[0], W64[:, k])


def test_gemm_row_subset_matches_full():
    rng = np.random.default_rng(12)
    N, K = 9, 256
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    scales = _np_f16_bits(rng.uniform(0.01, 0.1, (N, K // 64)))
    X = _bf16_bits(rng.standard_normal((2, K)))
    packed = oracle.pack(codes)
    Yf, Af = oracle.gemm(packed, scales, X)
    rows = np.array([8, 0, 3])
    Ys, As = oracle.gemm(packed, scales, X, rows=rows)
    assert np.array_equal(Ys, Yf[:, rows]) and np.array_equal(As, Af[:, rows])


def test_tolerance_helper():
    y_ref = np.array([1.0, -2.0, 0.0])
    absum = np.array([10.0, 10.0, 0.0])
    ok = oracle.within_tolerance(y_ref + np.array([0.0199, -0.0201, 9e-6]), y_ref, absum)
    assert list(ok) == [True, False, True]
