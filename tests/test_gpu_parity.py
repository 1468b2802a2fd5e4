"""GPU parity: libnf4 (through its C ABI, via the ctypes binding) against the CPU
oracle on the same seeded inputs.

Bars: nf4_pack codes and scales and nf4_unpack values bit-exact; products within
|y - y_ref| <= 2e-3 * sum_k |w~ x| + 1e-5 per element (y_ref, the bound and the
oracle's own codes all come from oracle/ on host copies of the generated
inputs, never from the GPU).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

import gpu_guard as guard

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def nf4():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dequant_gemv_nf4_amd as m
    m._lib._load()  # fail loudly if the library is missing
    return m


def _host_pack(W):
    packed, scales, st = oracle.quantize_pack(W.detach().cpu().numpy())
    return packed, scales, st


def _check_product(Y_gpu, Y_ref, A, what):
    Y = Y_gpu.detach().cpu().numpy().astype(np.float64).reshape(Y_ref.shape)
    ok = oracle.within_tolerance(Y, Y_ref, A)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        det = [(tuple(i), Y[tuple(i)], Y_ref[tuple(i)], A[tuple(i)]) for i in idx]
        pytest.fail(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance, e.g. {det}")


def _pack_gpu(nf4, W):
    N, K = W.shape
    cbuf, codes = guard.alloc((N, K // 2), torch.uint8, W.device)
    sbuf, scales = guard.alloc((N, K // 64), torch.int16, W.device)
    st = torch.full((1,), -7, dtype=torch.int32, device=W.device)
    nf4.nf4_pack(W, codes, scales, st)
    torch.cuda.synchronize()
    guard.check(cbuf, "pack codes")
    guard.check(sbuf, "pack scales")
    return codes, scales, int(st.item())


def _guarded_product(nf4, codes, scales, X, via_gemv=False):
    """Y = X . dequant^T through the C ABI (gemv, small-batch with a workspace
    where the plan splits, or prefill tiles beyond 32 rows), with guard bands
    around Y and the workspace."""
    M, K = X.shape
    N = codes.shape[0]
    ybuf, Y = guard.alloc((M, N), torch.float32, X.device)
    wbuf = None
    if via_gemv:
        nf4.nf4_gemv(codes, scales, X[0], Y.view(-1))
    else:
        big = M > nf4.MAX_M
        need = (nf4.prefill_workspace_bytes if big else nf4.smallm_workspace_bytes)(N, K, M)
        ws = None
        if need:
            wbuf, ws = guard.alloc(need, torch.uint8, X.device, fill=0)
            wbuf[:guard.GUARD] = guard.SENTINEL
            wbuf[guard.GUARD + need:] = guard.SENTINEL
        (nf4.nf4_gemm_prefill_ws if big else nf4.nf4_gemm_smallm_ws)(codes, scales, X, Y, ws)
    torch.cuda.synchronize()
    guard.check(ybuf, f"Y of M={M} N={N} K={K}")
    if wbuf is not None:
        guard.check(wbuf, f"workspace of M={M} N={N} K={K}")
    return Y


def _u16(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ packing
@pytest.mark.parametrize("N,K,sigma", [(1, 64, 0.02), (3, 128, 1.0), (17, 192, 0.02),
                                       (64, 4096, 0.02), (5, 11008, 0.015), (2, 32768, 3.0)])
def test_pack_bit_exact(nf4, N, K, sigma):
    W = wl.weights(N, K, sigma, seed=1000 + N * 7 + K, device=DEV)
    codes, scales, st = _pack_gpu(nf4, W)
    ref_p, ref_s, ref_st = _host_pack(W)
    assert st == ref_st == 0
    assert np.array_equal(codes.cpu().numpy(), ref_p)
    assert np.array_equal(_u16(scales), ref_s)


def test_pack_adversarial_values(nf4):
    """Decision boundaries and their fp32 neighbours, zero and tiny groups, huge and
    subnormal-scale groups; flagged groups (NaN, inf, overflow) and the status word."""
    _, l32 = oracle.codebook()
    mids = (l32[:-1].astype(np.float64) + l32[1:].astype(np.float64)) / 2
    row = []
    for m in mids:
        f = np.float32(m)
        row += [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2)), -f]
    row += [0.0, -0.0, 1.0, -1.0]
    row = np.array(row, np.float32)
    W = np.zeros((6, 128), np.float32)
    W[0, :len(row[:64])] = row[:64]
    W[0, 63] = 1.0
    W[0, 64:64 + len(row[64:])] = row[64:]
    W[0, 127] = -1.0
    W[1, :64] = 0.0                                  # zero group -> s = 0, codes 7
    W[1, 64:] = np.float32(2.0 ** -26)               # rounds to s = 0
    rng = np.random.default_rng(99)
    W[2, :64] = (rng.standard_normal(64) * 3e-6).astype(np.float32)   # subnormal fp16 scale
    W[2, 64:] = (rng.standard_normal(64) * 2e4).astype(np.float32)    # large, still finite
    W[3, :64] = np.float32(65519.0)                  # largest absmax that fits
    W[3, 64:] = (rng.standard_normal(64)).astype(np.float32)
    W[4, :] = 0.5
    W[4, 5] = np.nan                                 # non-finite -> flagged group
    W[5, :64] = 0.25
    W[5, 64:] = 0.5
    W[5, 100] = 70000.0                              # overflow -> flagged group
    Wg = torch.from_numpy(W).to(DEV)
    codes, scales, st = _pack_gpu(nf4, Wg)
    ref_p, ref_s, ref_st = oracle.quantize_pack(W)
    assert st == ref_st == (oracle.STATUS_NONFINITE | oracle.STATUS_SCALE_OVERFLOW)
    assert np.array_equal(codes.cpu().numpy(), ref_p)
    assert np.array_equal(_u16(scales), ref_s)
    # without a status word the call still packs identically
    codes2, scales2 = nf4.empty_packed(6, 128, DEV)
    nf4.nf4_pack(Wg, codes2, scales2, None)
    torch.cuda.synchronize()
    assert torch.equal(codes2, codes) and torch.equal(scales2, scales)


@pytest.mark.parametrize("N,K", [(7, 64), (33, 320), (128, 4096)])
def test_unpack_bit_exact(nf4, N, K):
    W = wl.weights(N, K, 0.02, seed=77 + N, device=DEV)
    ref_p, ref_s, _ = _host_pack(W)
    codes = torch.from_numpy(ref_p).to(DEV)
    scales = torch.from_numpy(ref_s.view(np.int16)).to(DEV)
    wbuf, Wt = guard.alloc((N, K), torch.float32, DEV)
    nf4.nf4_unpack(codes, scales, Wt)
    torch.cuda.synchronize()
    guard.check(wbuf, "unpack W_out")
    ref = oracle.dequant_f32(ref_p, ref_s)
    assert np.array_equal(Wt.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ products
def _product_case(nf4, M, N, K, sigma=0.02, seed=0, via_gemv=None):
    W = wl.weights(N, K, sigma, seed=seed * 1009 + N * 31 + K, device=DEV)
    X = wl.activations(M, K, seed=seed * 2003 + M * 17 + K, device=DEV)
    codes, scales, st = _pack_gpu(nf4, W)
    ref_p, ref_s, _ = _host_pack(W)
    assert np.array_equal(codes.cpu().numpy(), ref_p)
    Y = _guarded_product(nf4, codes, scales, X, via_gemv or (via_gemv is None and M == 1))
    Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(X))
    _check_product(Y, Yr, A, f"M={M} N={N} K={K}")
    return codes, scales, X, Y


@pytest.mark.parametrize("N", [1, 15, 16, 17, 300, 1024])
@pytest.mark.parametrize("K", [64, 128, 4096, 5120, 11008])
def test_gemv_shape_sweep(nf4, N, K):
    _product_case(nf4, 1, N, K)


def test_gemv_single_4096(nf4):
    """The single 4096 x 4096 GEMV workload, every output checked."""
    _product_case(nf4, 1, 4096, 4096, seed=1)


def test_gemv_large_k_and_ragged(nf4):
    _product_case(nf4, 1, 33, 32768)
    _product_case(nf4, 1, 129, 28672)
    _product_case(nf4, 1, 4099, 64)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 31, 32])
def test_gemm_smallm_m_sweep(nf4, M):
    _product_case(nf4, M, 272, 1024, seed=M)


@pytest.mark.parametrize("M,N,K", [(4, 33, 14336), (8, 100, 4096), (32, 48, 14336),
                                   (5, 20, 20480), (8, 17, 64), (32, 1, 128), (16, 4111, 192),
                                   (32, 40, 320), (24, 300, 2048)])
def test_gemm_smallm_shapes(nf4, M, N, K):
    _product_case(nf4, M, N, K, seed=3)


@pytest.mark.parametrize("M,N,K", [(3, 300, 256), (4, 1, 256), (8, 8, 1024), (8, 300, 512),
                                   (4, 4111, 3328), (3, 8, 1024), (4, 5120, 1024),
                                   (6, 4097, 1024), (5, 4111, 3328), (7, 12304, 2048),
                                   (8, 28688, 768)])
def test_gemm_quad_steps(nf4, M, N, K):
    """M <= 8 with K a multiple of 256 runs four groups per step: one step per
    row (K = 256: seven of the eight waves idle), step counts the eight waves do
    not share evenly (K = 768, 3328), fewer rows than a tile, rows past N in the
    last tile, and 2, 4 column tiles per workgroup with a ragged last group."""
    _product_case(nf4, M, N, K, seed=4)


@pytest.mark.parametrize("M,N,K", [(4, 16400, 1024), (8, 8200, 8192), (5, 4200, 5120),
                                   (8, 32768, 256), (6, 32784, 512), (7, 4113, 2048),
                                   (9, 12296, 4096), (16, 20000, 1280), (17, 28672, 2048),
                                   (32, 12290, 512), (24, 8200, 4096)])
def test_gemm_streaming_form(nf4, M, N, K):
    """More 16-column tiles than CUs run the streaming form: M = 4 above 16384
    rows (taken from the vector-ALU kernel), 4 steps per wave and 3 tiles per
    workgroup with a partial last tile, slices of 2 and 3 steps (K = 5120), one
    step in all (K = 256: seven slices empty) with 8 tiles per workgroup, 9 tiles
    per workgroup (past the form's limit: quad steps), a last tile of one row;
    above M = 8 one full 16-row tile (M = 9, 16, with slices of 1 and 2 steps)
    and two (M = 17, 24, 32), with partial last tiles of 8 and 2 rows."""
    _product_case(nf4, M, N, K, seed=5)


def test_gemm_quad_shape_with_scales_only_4_byte_aligned(nf4):
    """Scales 4 but not 8 bytes aligned: the quad-step shape falls back to the
    pair-step kernel, without a K-split (the workspace planned for the streaming
    form's split, which needs 8-byte aligned scales, goes unused)."""
    M, N, K = 8, 96, 14336
    W = wl.weights(N, K, 0.02, seed=61, device=DEV)
    codes, scales = _pack_gpu(nf4, W)[:2]
    buf = torch.zeros(N * (K // 64) + 2, dtype=torch.int16, device=DEV)
    buf[2:].copy_(scales.view(-1))
    sc = buf[2:].view(N, K // 64)
    assert sc.data_ptr() % 8 == 4
    X = wl.activations(M, K, seed=71, device=DEV)
    Y = nf4.gemm(codes, sc, X)
    torch.cuda.synchronize()
    Yr, A = oracle.gemm(codes.cpu().numpy(), _u16(scales), wl.bf16_bits(X))
    _check_product(Y.reshape(M, N), Yr, A, "scales 4-byte aligned, M=8")


def test_product_exact_identities(nf4):
    N, K = 300, 1024
    W = wl.weights(N, K, 0.02, seed=5, device=DEV)
    codes, scales, _ = _pack_gpu(nf4, W)
    for M in (1, 4, 8, 32):
        X = wl.activations(M, K, seed=6, device=DEV)
        Y = nf4.gemm(codes, scales, X)
        # zero activations -> exactly zero
        Z = nf4.gemm(codes, scales, torch.zeros_like(X))
        # power-of-two scaling commutes bitwise
        Y4 = nf4.gemm(codes, scales, (X.float() * 4.0).to(torch.bfloat16))
        Yq = nf4.gemm(codes, scales, (X.float() * 0.25).to(torch.bfloat16))
        # the same call twice -> the same bits
        Y2 = nf4.gemm(codes, scales, X)
        torch.cuda.synchronize()
        assert torch.all(Z == 0), M
        assert torch.equal(Y4, Y * 4.0), M
        assert torch.equal(Yq, Y * 0.25), M
        assert torch.equal(Y2, Y), M
    # every code the zero level -> y = 0
    zc = torch.full_like(codes, 0x77)
    X = wl.activations(8, K, seed=7, device=DEV)
    assert torch.all(nf4.gemm(zc, scales, X) == 0)
    assert torch.all(nf4.gemv(zc, scales, X[0]) == 0)


def test_activation_range_extremes(nf4):
    """Activations far outside the f16 range (huge, tiny, mixed) stay within tolerance."""
    N, K = 64, 2048
    W = wl.weights(N, K, 0.02, seed=8, device=DEV)
    codes, scales, _ = _pack_gpu(nf4, W)
    ref_p, ref_s, _ = _host_pack(W)
    for M in (1, 3, 8, 32):
        X = wl.activations(M, K, seed=9, device=DEV).float()
        X[0] *= 1e30
        if M > 1:
            X[1] *= 1e-30
        if M > 2:
            X[2, ::2] *= 1e6
        Xb = X.to(torch.bfloat16)
        Y = nf4.gemm(codes, scales, Xb)
        torch.cuda.synchronize()
        Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(Xb))
        _check_product(Y, Yr, A, f"range M={M}")


def _planted_range_case(nf4, M, N, K, ratios, units=None, seed=0, base=1.0):
    """Activations whose 32-value units each hold one entry `ratio` times larger
    than the rest, planted on a column whose weights are all exactly zero (code 7,
    the zero level): the small entries then carry the whole sum.  `units`
    restricts the planted units (default: every unit); ratios cycle over
    (row, unit); every activation is first multiplied by `base`."""
    W = wl.weights(N, K, 0.02, seed=seed * 101 + N + K, device=DEV).cpu()
    X = wl.activations(M, K, seed=seed * 103 + M + K).float() * base
    U = K // 32
    units = range(U) if units is None else units
    planted = []
    for m in range(M):
        for j, u in enumerate(units):
            k0 = 32 * u + (7 * u + 3 * m) % 32
            W[:, k0] = 0.0
            r = ratios[(j + m) % len(ratios)]
            X[m, k0] = (1.5 if (u + m) % 2 else -1.5) * r * base
            planted.append((m, k0))
    Xb = X.to(torch.bfloat16)
    for m, k0 in planted:  # the planted entry is the unit's largest, exactly
        assert abs(float(Xb[m, k0])) == abs(float(X[m, k0]))
    codes, scales, st = _pack_gpu(nf4, W.to(DEV))
    assert st == 0
    ref_p, ref_s, _ = _host_pack(W)
    assert np.array_equal(codes.cpu().numpy(), ref_p)
    assert np.all(oracle.unpack_codes(ref_p)[:, [k for _, k in planted]] == 7)
    Y = _guarded_product(nf4, codes, scales, Xb.to(DEV))
    Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(Xb))
    _check_product(Y, Yr, A, f"planted range M={M} N={N} K={K} ratios={ratios}")
    return Y, Yr


@pytest.mark.parametrize("M", [1, 2, 4])
def test_activation_range_planted_on_zero_weights(nf4, M):
    """Per-unit activation ranges of 2^20, 2^26 (held exactly by the per-unit f16
    shift) and 2^30, 2^40, 2^100 (beyond it: the exact fp32 form), with the large
    entry on a zero-level weight, at M = 1, 2 and 4 on 6144 rows (all three on
    the vector-ALU kernel)."""
    ratios = [2.0 ** 20, 2.0 ** 26, 2.0 ** 30, 2.0 ** 40, 2.0 ** 100]
    _planted_range_case(nf4, M, 6144, 4096, ratios, seed=M)
    # the same at a larger magnitude: the rest ~ 2^60, the planted entry 2^100
    # above the usual scale, so the sums stay within fp32 only if nothing is
    # summed before its scale is applied
    Y, Yr = _planted_range_case(nf4, M, 6144, 1024, [2.0 ** 40], seed=10 + M, base=2.0 ** 60)
    assert np.isfinite(Y.cpu().numpy()).all()


@pytest.mark.parametrize("M,N,K", [(8, 16400, 2048), (5, 20480, 1024), (16, 16400, 2048),
                                   (32, 20480, 1024), (24, 16400, 4096), (8, 8200, 4096)])
def test_streaming_form_activation_ranges(nf4, M, N, K):
    """From 5 tiles per workgroup the streaming MFMA form runs f16 products with
    one power-of-two shift per group of 64 k shared by every row: groups whose
    entries span more than f16 holds (planted 2^30, 2^40, 2^100 above the rest on
    zero-level weights, or rows 2^40 apart) go through its exact fp32 pass, the
    others through f16.  Shapes: the padded 8-row tile (M = 5, 8), one and two
    16-row tiles (M = 16; 24, 32), slices of one and two steps, some waves with
    none (K = 1024); and 3 tiles per workgroup, which stays on bf16 hi + lo."""
    U = K // 32
    ratios = [2.0 ** 20, 2.0 ** 26, 2.0 ** 30, 2.0 ** 40, 2.0 ** 100]
    # planted in every 16th unit: most groups exact in f16, the rest wide
    _planted_range_case(nf4, M, N, K, ratios, units=range(0, U, 16), seed=20 + M)
    # one row 2^40 below the others: every group is wide through the rows
    W = wl.weights(N, K, 0.02, seed=31 + M, device=DEV)
    X = wl.activations(M, K, seed=37 + M).float()
    X[M // 2] *= 2.0 ** -40
    Xb = X.to(torch.bfloat16)
    codes, scales, st = _pack_gpu(nf4, W)
    ref_p, ref_s, _ = _host_pack(W)
    Y = _guarded_product(nf4, codes, scales, Xb.to(DEV))
    Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(Xb))
    _check_product(Y, Yr, A, f"rows 2^40 apart M={M} N={N} K={K}")


def test_activation_range_in_one_slice_only(nf4):
    """K = 16384 at M = 1 runs four K-slices: only the waves whose slice holds a
    planted unit take the exact fp32 form, the others the f16 form; the slices'
    sums meet in one output."""
    U = 16384 // 32
    _planted_range_case(nf4, 1, 6144, 16384, [2.0 ** 40], units=range(0, U // 4, 16), seed=5)
    _planted_range_case(nf4, 1, 6144, 16384, [2.0 ** 30], units=[U - 1], seed=6)


def test_activation_range_with_bf16_subnormals(nf4):
    """bf16 subnormal activations beside normal ones in one unit (both forms of
    the per-unit check): within tolerance at M = 1, 2."""
    N, K = 6144, 2048
    W = wl.weights(N, K, 0.02, seed=31, device=DEV)
    codes, scales, _ = _pack_gpu(nf4, W)
    ref_p, ref_s, _ = _host_pack(W)
    for M in (1, 2):
        X = wl.activations(M, K, seed=32 + M).float()
        X[:, 5::64] = 3e-39   # subnormal in bf16 (below 2^-126)
        X[:, 9::128] *= 2.0 ** -100
        Xb = X.to(torch.bfloat16)
        Y = nf4.gemm(codes, scales, Xb.to(DEV))
        torch.cuda.synchronize()
        Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(Xb))
        _check_product(Y, Yr, A, f"subnormal activations M={M}")


# ------------------------------------------------------------------ full sizes, sampled rows
def _sampled_rows(N, count, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(count, N), replace=False).tolist())
    rows |= {0, N - 1}
    return np.array(sorted(rows), np.int64)


def _full_size_case(nf4, set_, proj, N, K, M):
    W = wl.weights(N, K, set_.sigma, wl.seed_for(set_.name, 0, proj, "W"), device=DEV)
    X = wl.activations(M, K, wl.seed_for(set_.name, 0, proj, "x"), device=DEV)
    codes, scales, st = _pack_gpu(nf4, W)
    assert st == 0
    Y = _guarded_product(nf4, codes, scales, X, via_gemv=M == 1)
    rows = _sampled_rows(N, 48, N + K + M)
    Wr = W[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    ref_p, ref_s, _ = oracle.quantize_pack(Wr)
    r = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(codes[r].cpu().numpy(), ref_p), f"{set_.name}/{proj} codes"
    assert np.array_equal(_u16(scales[r]), ref_s), f"{set_.name}/{proj} scales"
    Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(X))
    _check_product(Y.reshape(M, N)[:, r], Yr, A, f"{set_.name}/{proj} M={M}")
    del W


@pytest.mark.parametrize("set_", [wl.SET_7B, wl.SET_13B, wl.SET_70B, wl.SET_8B_SMALLM],
                         ids=lambda s: s.name)
def test_pack_first_middle_last_layers(nf4, set_):
    """Packing of layers 0, L/2 and L-1 of the set, each with its own seeds: 64
    random rows of every projection, plus the first and last row, bit-exact
    against the oracle's quantizer."""
    for layer in (0, set_.layers // 2, set_.layers - 1):
        for proj, N, K in set_.projections:
            W = wl.weights(N, K, set_.sigma, wl.seed_for(set_.name, layer, proj, "W"), device=DEV)
            codes, scales, st = _pack_gpu(nf4, W)
            assert st == 0
            r = torch.from_numpy(_sampled_rows(N, 64, 7919 * layer + N + K)).to(DEV)
            ref_p, ref_s, _ = oracle.quantize_pack(W[r].cpu().numpy())
            what = f"{set_.name} layer {layer} {proj}"
            assert np.array_equal(codes[r].cpu().numpy(), ref_p), what + " codes"
            assert np.array_equal(_u16(scales[r]), ref_s), what + " scales"
            del W, codes, scales


def test_pack_whole_matrices_of_a_7b_layer(nf4):
    """Every row of every projection of the 7B set's middle layer, bit-exact."""
    layer = wl.SET_7B.layers // 2
    for proj, N, K in wl.SET_7B.projections:
        W = wl.weights(N, K, wl.SET_7B.sigma, wl.seed_for(wl.SET_7B.name, layer, proj, "W"),
                       device=DEV)
        codes, scales, st = _pack_gpu(nf4, W)
        assert st == 0
        ref_p, ref_s, _ = oracle.quantize_pack(W.cpu().numpy())
        assert np.array_equal(codes.cpu().numpy(), ref_p), f"7B layer {layer} {proj} codes"
        assert np.array_equal(_u16(scales), ref_s), f"7B layer {layer} {proj} scales"
        del W, codes, scales


def _launch_shapes(set_):
    """(name, N, K) of every distinct product shape of a layer, one launch per
    projection and with same-x projections fused along N."""
    seen, out = set(), []
    for fused in (False, True):
        for name, projs in wl.launch_groups(set_, fused):
            N, K = sum(n for _, n, _ in projs), projs[0][2]
            if (N, K) not in seen:
                seen.add((N, K))
                out.append((name, N, K))
    return out


@pytest.mark.parametrize("set_", [wl.SET_7B, wl.SET_13B, wl.SET_70B], ids=lambda s: s.name)
def test_full_size_layer_shapes_m1(nf4, set_):
    for name, N, K in _launch_shapes(set_):
        _full_size_case(nf4, set_, name, N, K, 1)


# M = 2, 3, 4: the vector-ALU kernel on the wide matrices and the MFMA kernel on the
# 4096-row ones (both sides of the dispatch threshold); 8, 16, 32: the MFMA kernel
# with its K-split plans (through gemm(), which brings a workspace)
@pytest.mark.parametrize("M", [2, 3, 4, 8, 16, 32])
def test_full_size_smallm_8b(nf4, M):
    for name, N, K in _launch_shapes(wl.SET_8B_SMALLM):
        _full_size_case(nf4, wl.SET_8B_SMALLM, name, N, K, M)


def test_pack_into_row_slices_of_a_fused_matrix(nf4):
    """q, k, v packed one by one into row ranges of one buffer equal the oracle's
    packing of the concatenated matrix, and the fused product matches the oracle."""
    K, parts = 512, (96, 32, 32)
    Ws = [wl.weights(n, K, 0.02, seed=40 + i, device=DEV) for i, n in enumerate(parts)]
    codes, scales = nf4.empty_packed(sum(parts), K, DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    r0 = 0
    for W in Ws:
        nf4.nf4_pack(W, codes[r0:r0 + W.shape[0]], scales[r0:r0 + W.shape[0]], st)
        r0 += W.shape[0]
    torch.cuda.synchronize()
    ref_p, ref_s, _ = _host_pack(torch.cat(Ws))
    assert np.array_equal(codes.cpu().numpy(), ref_p)
    assert np.array_equal(_u16(scales), ref_s)
    x = wl.activations(1, K, seed=44, device=DEV)
    y = nf4.gemv(codes, scales, x[0])
    torch.cuda.synchronize()
    yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(x))
    _check_product(y.reshape(1, -1), yr, A, "fused q|k|v")


@pytest.mark.parametrize("M", [1, 8, 32])
def test_products_with_scales_only_2_byte_aligned(nf4, M):
    """Scales at an address that is 2 but not 4 bytes aligned (allowed by the ABI)
    take the 16-bit scale paths; results match the oracle."""
    N, K = 96, 1024
    W = wl.weights(N, K, 0.02, seed=60 + M, device=DEV)
    codes, scales = _pack_gpu(nf4, W)[:2]
    buf = torch.zeros(N * (K // 64) + 1, dtype=torch.int16, device=DEV)
    buf[1:].copy_(scales.view(-1))
    sc = buf[1:].view(N, K // 64)
    assert sc.data_ptr() % 4 == 2
    X = wl.activations(M, K, seed=70 + M, device=DEV)
    Y = nf4.gemv(codes, sc, X[0]) if M == 1 else nf4.gemm(codes, sc, X)
    torch.cuda.synchronize()
    Yr, A = oracle.gemm(codes.cpu().numpy(), _u16(scales), wl.bf16_bits(X))
    _check_product(Y.reshape(M, N), Yr, A, f"unaligned scales M={M}")
