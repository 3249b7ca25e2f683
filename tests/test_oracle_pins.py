"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against an independent implementation (scipy's
normal quantile, numpy's float16 conversion, numpy/BLAS products, Python's
exact rationals), a closed form, an invariant, or a hand-built example whose
answer follows from the pages' definitions:

- deep-fold "Decode V2", section 6 (Linear primitive): 16-float table times
  group scale times x; section 2: groups of 64 along K;
- golang.design accel/tensor, type Int4 (low nibble first), func Cast
  (f32 -> f16 nearest-even, overflow -> inf; bf16 -> f32 exact), func Argmax
  (ties to the lowest index).

No GPU is needed.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import ndtr, ndtri

import workloads as wl

DELTA = 0.5 * (1 / 30 + 1 / 32)


# --------------------------------------------------------------------------
# Codebook
# --------------------------------------------------------------------------

def _scipy_levels():
    """NF4 levels from scipy's inverse normal CDF on numpy's linspace grids."""
    top = 1 - DELTA
    pos = ndtri(np.linspace(top, 0.5, 9)[:-1])
    neg = -ndtri(np.linspace(top, 0.5, 8)[:-1])
    v = np.sort(np.concatenate([pos, neg, [0.0]])) / ndtri(top)
    return v


def test_codebook_matches_scipy_construction(oracle_mod):
    ours = oracle_mod.codebook_f32()
    ref = _scipy_levels().astype(np.float32)
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32)), (ours, ref)
    ours64 = oracle_mod.codebook_f64()
    assert np.max(np.abs(ours64 - _scipy_levels())) < 1e-14


def test_codebook_structure(oracle_mod):
    c = oracle_mod.codebook_f32()
    assert c.size == 16
    assert c[0] == -1.0 and c[15] == 1.0
    assert c.view(np.uint32)[7] == 0  # +0.0 exactly
    assert np.all(np.diff(c.astype(np.float64)) > 0)
    assert np.sum(c < 0) == 7 and np.sum(c > 0) == 8


def test_codebook_levels_are_normal_quantiles(oracle_mod):
    # Forward check with the CDF: level * Phi^-1(1-delta) sits at the grid
    # probability the construction names.
    c = oracle_mod.codebook_f64()
    top = ndtri(1 - DELTA)
    p_pos = ndtr(c[8:] * top)
    grid_pos = (1 - DELTA) - np.arange(7, -1, -1) * ((1 - DELTA) - 0.5) / 8
    assert np.allclose(p_pos, grid_pos, rtol=0, atol=1e-14)
    p_neg = ndtr(-c[:7] * top)
    grid_neg = (1 - DELTA) - np.arange(0, 7) * ((1 - DELTA) - 0.5) / 7
    assert np.allclose(p_neg, grid_neg, rtol=0, atol=1e-14)


@pytest.mark.parametrize("p", [1e-12, 1e-6, 0.01, 0.2, 0.5, 0.5 + 1e-9, 0.7, 0.9677, 0.999, 1 - 1e-9])
def test_phi_inv_against_scipy(oracle_mod, p):
    z = oracle_mod.phi_inv(p)
    assert abs(z - ndtri(p)) <= 1e-13 * max(1.0, abs(z))


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def _f16_bits_numpy(v):
    with np.errstate(over="ignore"):
        return np.asarray(v, np.float32).astype(np.float16).view(np.uint16)


def test_f32_to_f16_rne_matches_numpy_on_structured_values(oracle_mod):
    all_h = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    hv = all_h.view(np.float16).astype(np.float32)
    finite = np.isfinite(hv)
    hv = hv[finite]
    # every half value, its fp32 neighbours, and the midpoints between
    # consecutive halves (the ties) with their fp32 neighbours
    pos = np.sort(np.unique(np.abs(hv)))
    mids = ((pos[:-1].astype(np.float64) + pos[1:].astype(np.float64)) / 2).astype(np.float32)
    cand = np.concatenate([hv, mids, -mids])
    cand = np.concatenate([cand, np.nextafter(cand, np.float32(np.inf)),
                           np.nextafter(cand, np.float32(-np.inf))])
    extra = np.array([0.0, -0.0, 65504, 65519.996, 65520, 65536, 1e38, np.inf, -np.inf,
                      2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26, 1e-30,
                      2.0 ** -14, 2.0 ** -14 - 2.0 ** -25], np.float32)
    cand = np.concatenate([cand, extra, -extra])
    ours = oracle_mod.f32_to_f16_bits(cand)
    ref = _f16_bits_numpy(cand)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(cand[i]), hex(ours[i]), hex(ref[i])) for i in bad[:10]]


def test_f32_to_f16_rne_matches_numpy_random(oracle_mod):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    assert np.array_equal(oracle_mod.f32_to_f16_bits(v), _f16_bits_numpy(v))
    # values concentrated in the half range, where rounding matters
    v2 = (rng.standard_normal(1 << 20) * np.exp2(rng.integers(-26, 17, 1 << 20))).astype(np.float32)
    assert np.array_equal(oracle_mod.f32_to_f16_bits(v2), _f16_bits_numpy(v2))


def test_f32_to_f16_nan_stays_nan(oracle_mod):
    h = oracle_mod.f32_to_f16_bits([np.nan])[0]
    assert (h & 0x7c00) == 0x7c00 and (h & 0x3ff) != 0


def test_f16_to_f64_all_patterns(oracle_mod):
    h = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    ours = oracle_mod.f16_bits_to_f64(h)
    ref = h.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(ours[m], ref[m])
    assert np.array_equal(np.signbit(ours[m]), np.signbit(ref[m]))


def test_bf16_to_f64_all_patterns(oracle_mod):
    b = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    ours = oracle_mod.bf16_bits_to_f64(b)
    ref = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    m = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[m], ref[m])


# --------------------------------------------------------------------------
# Pack
# --------------------------------------------------------------------------

def _unpack_codes(codes, M, K):
    """Codes [M, K] from the packed bytes, low nibble = even k (accel/tensor
    type Int4)."""
    lo = codes & 0xF
    hi = codes >> 4
    out = np.empty((M, K), np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def _edge_matrix():
    """64-row, 256-column matrix mixing ordinary and degenerate blocks."""
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    W[0, :64] = 0.0                     # zero block
    W[1, :64] = -0.0                    # negative-zero block
    W[2, :64] = 1e-9                    # absmax below half the smallest fp16 subnormal
    W[3, :64] = rng.standard_normal(64) * 1e-6   # subnormal fp16 scale
    W[4, :64] = rng.standard_normal(64) * 1e3    # large scale
    W[5, 64:128] = 65519.0              # rounds to 65504
    W[6, :64] = rng.standard_normal(64).astype(np.float32) * np.float32(2.0 ** -14)
    W[7, :] = np.exp2(rng.integers(-30, 10, 256)).astype(np.float32) * np.sign(rng.standard_normal(256)).astype(np.float32)
    W[8, :64] = 0.0
    W[8, 5] = 1.0                       # one nonzero in a block
    W[9, :64] = 1.0                     # constant block
    W[10, :64] = -1.0
    return W


def test_scale_is_fp16_rne_of_block_absmax(oracle_mod):
    for W in (wl.weights(256, 512, 0), _edge_matrix()):
        M, K = W.shape
        _, scales, st = oracle_mod.pack(W)
        assert st == 0
        amax = np.abs(W.reshape(M, K // 64, 64)).max(axis=2)
        assert np.array_equal(scales, _f16_bits_numpy(amax))


def _nearest_check(W, codes, scales, cb):
    """Every chosen level is a nearest level to w/s (exact arithmetic decides
    near-ties); an exact midpoint goes to the lower level."""
    M, K = W.shape
    code = _unpack_codes(codes, M, K)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 64, axis=1)
    w = W.astype(np.float64)
    lv = cb.astype(np.float64)
    d = np.abs(w[..., None] - lv[None, None, :] * s[..., None])  # [M,K,16]
    chosen = np.take_along_axis(d, code[..., None], axis=2)[..., 0]
    best = d.min(axis=2)
    zero_s = s == 0
    assert np.all(code[zero_s] == 7)
    suspicious = np.nonzero(~zero_s & (chosen > best * (1 + 1e-9)))
    assert suspicious[0].size == 0, "chosen level is not nearest"
    # near-ties: settle exactly with rationals
    close = np.nonzero(~zero_s & (np.sort(d, axis=2)[..., 1] <= best * (1 + 1e-9)))
    for m, k in zip(*close):
        wf = Fraction(float(W[m, k]))
        sf = Fraction(float(s[m, k]))
        dist = [abs(wf - Fraction(float(c)) * sf) for c in cb]
        dmin = min(dist)
        nearest = [j for j in range(16) if dist[j] == dmin]
        assert code[m, k] == min(nearest), (m, k, nearest, code[m, k])


def test_pack_chooses_nearest_level_brute_force(oracle_mod):
    cb = oracle_mod.codebook_f32()
    for W in (wl.weights(256, 512, 0), _edge_matrix()):
        codes, scales, st = oracle_mod.pack(W)
        assert st == 0
        _nearest_check(W, codes, scales, cb)


def test_pack_tie_goes_to_lower_level(oracle_mod):
    cb = oracle_mod.codebook_f32().astype(np.float64)
    tried = 0
    for i in range(15):
        mid = Fraction(float(cb[i])) / 2 + Fraction(float(cb[i + 1])) / 2
        mf = np.float32(float(mid))
        if Fraction(float(mf)) != mid:
            continue  # midpoint not representable in fp32 at scale 1
        tried += 1
        W = np.zeros((1, 64), np.float32)
        W[0, 0] = 1.0          # pins the scale to exactly 1.0
        W[0, 1] = mf
        W[0, 2] = np.nextafter(mf, np.float32(np.inf))
        W[0, 3] = np.nextafter(mf, np.float32(-np.inf))
        codes, scales, st = oracle_mod.pack(W)
        code = _unpack_codes(codes, 1, 64)[0]
        assert scales[0, 0] == 0x3C00
        assert code[1] == i and code[2] == i + 1 and code[3] == i
    assert tried >= 3


def test_pack_nibble_order_and_layout_hand_built(oracle_mod):
    # Weights placed exactly on levels (scale 1) so every code is known; the
    # expected bytes are written from the rule: byte j = code 2j | code 2j+1 << 4.
    cb = oracle_mod.codebook_f32()
    M, K = 3, 192
    want = np.zeros((M, K), np.int64)
    for m in range(M):
        for k in range(K):
            want[m, k] = (3 * m + 5 * k + (k // 64)) % 16
        for b in range(K // 64):
            want[m, b * 64] = 15  # absmax 1.0 in every block -> scale exactly 1
    W = cb[want].astype(np.float32)
    codes, scales, st = oracle_mod.pack(W)
    assert st == 0
    assert np.all(scales == 0x3C00)
    for m in range(M):
        for j in range(K // 2):
            assert codes[m, j] == (want[m, 2 * j] | (want[m, 2 * j + 1] << 4))
    # one concrete byte spelled out: codes 3 then 12 give 0xC3
    W2 = np.zeros((1, 64), np.float32)
    W2[0, 0], W2[0, 1], W2[0, 2] = cb[3], cb[12], 1.0
    c2, _, _ = oracle_mod.pack(W2)
    assert c2[0, 0] == 0xC3 and c2[0, 1] == 0x7F


def test_pack_zero_and_degenerate_blocks(oracle_mod):
    W = _edge_matrix()
    codes, scales, st = oracle_mod.pack(W)
    assert st == 0
    for m in (0, 1, 2):
        assert scales[m, 0] == 0
        assert np.all(codes[m, :32] == 0x77)
    assert 0 < scales[3, 0] < 0x0400  # subnormal fp16 scale
    assert scales[5, 1] == 0x7BFF       # 65519 -> 65504
    # a lone nonzero in a zero block: it is the absmax, so level +1, the rest 0
    code = _unpack_codes(codes, 64, 256)
    assert code[8, 5] == 15 and np.all(np.delete(code[8, :64], 5) == 7)
    assert np.all(code[9, :64] == 15) and np.all(code[10, :64] == 0)


def test_pack_refuses_nonfinite_and_overflow(oracle_mod):
    W = np.zeros((2, 128), np.float32)
    W[0, 3] = np.nan
    assert oracle_mod.pack(W)[2] == oracle_mod.PACK_NONFINITE
    W[0, 3] = np.inf
    assert oracle_mod.pack(W)[2] == oracle_mod.PACK_NONFINITE
    W[0, 3] = 0
    W[1, 100] = -65520.0
    assert oracle_mod.pack(W)[2] == oracle_mod.PACK_OVERFLOW
    W[0, 3] = -np.inf
    assert oracle_mod.pack(W)[2] == oracle_mod.PACK_NONFINITE | oracle_mod.PACK_OVERFLOW
    W[:] = 0
    W[1, 100] = 65519.99
    assert oracle_mod.pack(W)[2] == 0


def test_pack_idempotent_through_dequant(oracle_mod):
    for W in (wl.weights(256, 512, 0), _edge_matrix()):
        M, K = W.shape
        codes, scales, _ = oracle_mod.pack(W)
        W2 = oracle_mod.dequant(codes, scales, M, K).astype(np.float32)
        codes2, scales2, st = oracle_mod.pack(W2)
        assert st == 0
        assert np.array_equal(codes, codes2) and np.array_equal(scales, scales2)


@pytest.mark.parametrize("j", [-3, -1, 1, 4])
def test_pack_scale_linearity(oracle_mod, j):
    W = wl.weights(64, 512, 5)
    codes, scales, _ = oracle_mod.pack(W)
    codes2, scales2, st = oracle_mod.pack((W * np.float32(2.0 ** j)).astype(np.float32))
    assert st == 0
    assert np.array_equal(codes, codes2)
    s1 = scales.view(np.float16).astype(np.float64)
    s2 = scales2.view(np.float16).astype(np.float64)
    assert np.array_equal(s2, s1 * 2.0 ** j)


def test_pack_error_bound_closed_form(oracle_mod):
    # |w - What| is at most half the widest gap between neighbouring levels,
    # times s, plus the amount by which |w| may exceed s after rounding.
    cb = oracle_mod.codebook_f32().astype(np.float64)
    half_gap = np.max(np.diff(cb)) / 2
    assert abs(half_gap - (cb[1] - cb[0]) / 2) < 1e-15  # widest gap is the first
    W = wl.weights(256, 2048, 6)
    M, K = W.shape
    codes, scales, _ = oracle_mod.pack(W)
    What = oracle_mod.dequant(codes, scales, M, K)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 64, axis=1)
    err = np.abs(W.astype(np.float64) - What)
    bound = half_gap * s + np.maximum(0.0, np.abs(W) - s)
    assert np.all(err <= bound * (1 + 1e-12))
    assert np.max(err / s) > 0.9 * half_gap  # and the bound is nearly attained


def test_pack_row_ranges_compose(oracle_mod):
    W = wl.weights(97, 256, 9)
    c1, s1, _ = oracle_mod.pack(W, threads=1)
    c4, s4, _ = oracle_mod.pack(W, threads=4)
    assert np.array_equal(c1, c4) and np.array_equal(s1, s4)


# --------------------------------------------------------------------------
# Dequant, GEMV, GEMM
# --------------------------------------------------------------------------

def test_dequant_hand_built_bytes(oracle_mod):
    cb = oracle_mod.codebook_f32().astype(np.float64)
    codes = np.zeros((2, 64), np.uint8)
    codes[0, 0] = 0xC3
    codes[1, 33] = 0x5A
    scales = np.array([[0x3C00, 0x4000], [0x3800, 0xC000]], np.uint16)  # 1, 2, 0.5, -2
    What = oracle_mod.dequant(codes, scales, 2, 128)
    assert What[0, 0] == cb[3] * 1.0 and What[0, 1] == cb[12] * 1.0
    assert What[0, 2] == cb[0] * 1.0 and What[0, 64] == cb[0] * 2.0
    assert What[1, 66] == cb[0xA] * -2.0 and What[1, 67] == cb[0x5] * -2.0
    assert What[1, 0] == cb[0] * 0.5


def _fixture(M, K, seed, xrec="normal"):
    W = wl.weights(M, K, seed)
    x = wl.activation(K, seed, xrec)
    return W, x


def test_gemv_matches_blas_on_dequant(oracle_mod):
    for (M, K, seed) in [(256, 512, 0), (37, 1280, 12), (5, 11008, 13)]:
        W, x = _fixture(M, K, seed)
        codes, scales, _ = oracle_mod.pack(W)
        y, S = oracle_mod.gemv(codes, scales, M, K, x)
        What = oracle_mod.dequant(codes, scales, M, K)
        xv = wl.bf16_bits_to_f32(x).astype(np.float64)
        ref = What @ xv
        assert np.all(np.abs(y - ref) <= 1e-12 * np.abs(What) @ np.abs(xv))
        assert np.allclose(S, np.abs(What) @ np.abs(xv), rtol=1e-12, atol=0)


def test_gemv_exact_rational_tiny(oracle_mod):
    M, K = 4, 128
    W, x = _fixture(M, K, 21)
    codes, scales, _ = oracle_mod.pack(W)
    y, S = oracle_mod.gemv(codes, scales, M, K, x)
    cb = oracle_mod.codebook_f32()
    code = _unpack_codes(codes, M, K)
    xv = wl.bf16_bits_to_f32(x)
    for m in range(M):
        exact = Fraction(0)
        for k in range(K):
            s = Fraction(float(scales[m, k // 64:k // 64 + 1].view(np.float16)[0]))
            exact += Fraction(float(cb[code[m, k]])) * s * Fraction(float(xv[k]))
        assert abs(Fraction(y[m]) - exact) <= Fraction(K * 2.0 ** -53) * Fraction(S[m])


def test_gemv_one_hot_x_selects_column(oracle_mod):
    M, K = 64, 256
    W, _ = _fixture(M, K, 22)
    codes, scales, _ = oracle_mod.pack(W)
    What = oracle_mod.dequant(codes, scales, M, K)
    for k in (0, 1, 63, 64, 201, 255):
        x = np.zeros(K, np.uint16)
        x[k] = 0x3F80  # bf16 1.0
        y, _ = oracle_mod.gemv(codes, scales, M, K, x)
        assert np.array_equal(y, What[:, k])


def test_gemv_constant_code_closed_form(oracle_mod):
    cb = oracle_mod.codebook_f32().astype(np.float64)
    M, K = 16, 256
    rng = np.random.default_rng(3)
    scales = _f16_bits_numpy(rng.uniform(0.01, 2, (M, K // 64)))
    x = np.full(K, 0x3F80, np.uint16)
    for j in (0, 3, 7, 12, 15):
        codes = np.full((M, K // 2), j | (j << 4), np.uint8)
        y, _ = oracle_mod.gemv(codes, scales, M, K, x)
        sums = scales.view(np.float16).astype(np.float64).sum(axis=1)
        assert np.allclose(y, cb[j] * 64 * sums, rtol=1e-14, atol=0)
        if j == 7:
            assert np.all(y == 0)


def test_gemv_zero_block_contributes_nothing(oracle_mod):
    M, K = 32, 512
    W, x = _fixture(M, K, 23)
    codes, scales, _ = oracle_mod.pack(W)
    y0, _ = oracle_mod.gemv(codes, scales, M, K, x)
    W[:, 128:192] = 0
    codes2, scales2, _ = oracle_mod.pack(W)
    y1, _ = oracle_mod.gemv(codes2, scales2, M, K, x)
    x2 = x.copy()
    x2[128:192] = 0
    y2, _ = oracle_mod.gemv(codes, scales, M, K, x2)
    assert np.allclose(y1, y2, rtol=1e-13, atol=1e-15)
    assert not np.allclose(y0, y1)


def test_gemv_linearity_bit_exact(oracle_mod):
    M, K = 64, 1024
    W, x = _fixture(M, K, 24)
    codes, scales, _ = oracle_mod.pack(W)
    y, S = oracle_mod.gemv(codes, scales, M, K, x)
    x2 = (x.astype(np.uint32) + (2 << 7)).astype(np.uint16)  # exponent + 2: x * 4 (normal x)
    y2, S2 = oracle_mod.gemv(codes, scales, M, K, x2)
    assert np.array_equal(y2, 4 * y) and np.array_equal(S2, 4 * S)
    s2 = (scales.astype(np.uint32) + (1 << 10)).astype(np.uint16)  # scales * 2 (normal)
    y3, _ = oracle_mod.gemv(codes, s2, M, K, x)
    assert np.array_equal(y3, 2 * y)


def test_gemv_row_range_and_list(oracle_mod):
    M, K = 300, 256
    W, x = _fixture(M, K, 25)
    codes, scales, _ = oracle_mod.pack(W)
    y, S = oracle_mod.gemv(codes, scales, M, K, x)
    yt, St = oracle_mod.gemv(codes, scales, M, K, x, threads=3)
    assert np.array_equal(y, yt) and np.array_equal(S, St)
    rows = [299, 0, 17, 150]
    yl, Sl = oracle_mod.gemv_row_list(codes, scales, M, K, x, rows)
    assert np.array_equal(yl, y[rows]) and np.array_equal(Sl, S[rows])


def test_gemm_matches_blas_and_gemv(oracle_mod):
    M, K, N = 96, 640, 5
    W = wl.weights(M, K, 26)
    X = wl.activations(N, K, 26, "unit_rms")
    codes, scales, _ = oracle_mod.pack(W)
    Y, S = oracle_mod.gemm(codes, scales, M, K, X)
    What = oracle_mod.dequant(codes, scales, M, K)
    Xv = wl.bf16_bits_to_f32(X).astype(np.float64)
    ref = Xv @ What.T
    assert np.all(np.abs(Y - ref) <= 1e-12 * (np.abs(Xv) @ np.abs(What).T))
    for n in range(N):
        yn, Sn = oracle_mod.gemv(codes, scales, M, K, X[n])
        assert np.array_equal(Y[n], yn) and np.array_equal(S[n], Sn)


# --------------------------------------------------------------------------
# Argmax and the acceptance bound
# --------------------------------------------------------------------------

def test_argmax_ties_lowest_index_and_nan(oracle_mod):
    y = np.array([1.0, 3.0, 2.0, 3.0, 3.0], np.float64)
    assert oracle_mod.argmax(y) == 1
    assert oracle_mod.argmax(y.astype(np.float32)) == 1
    y = np.array([np.nan, -5.0, np.nan, -5.0], np.float32)
    assert oracle_mod.argmax(y) == 1
    assert oracle_mod.argmax(np.zeros(0)) == -1
    rng = np.random.default_rng(1)
    for _ in range(20):
        v = rng.integers(0, 7, 1000).astype(np.float64)  # many ties
        assert oracle_mod.argmax(v) == int(np.argmax(v))


def test_within_tolerance_bound():
    import oracle
    ok, r = oracle.within_tolerance([1.0 + 1e-5], np.array([1.0]), np.array([10.0]))
    assert ok and r < 1
    ok, r = oracle.within_tolerance([1.0 + 0.02], np.array([1.0]), np.array([10.0]))
    assert not ok and r > 1
    ok, _ = oracle.within_tolerance([np.nan], np.array([1.0]), np.array([10.0]))
    assert not ok


# --------------------------------------------------------------------------
# Fused-projection epilogue: SiLU, SwiGLU, bias and residual
# --------------------------------------------------------------------------

def test_silu_odd_part_identity(oracle_mod):
    # silu(z) - silu(-z) = z (sigma(z) + sigma(-z) = 1): fixes the sign of
    # the exponent and which factor is the sigmoid.
    for z in (0.25, 1.0, 2.5, -3.0, 7.0, 0.0):
        assert abs((oracle_mod.silu(z) - oracle_mod.silu(-z)) - z) <= 4e-16 * max(1.0, abs(z))


def test_silu_limits_and_minimum(oracle_mod):
    assert oracle_mod.silu(0.0) == 0.0
    assert oracle_mod.silu(40.0) == 40.0            # sigmoid(40) rounds to 1 in fp64
    assert -1e-15 < oracle_mod.silu(-40.0) < 0.0    # -40 e^-40
    # The minimum of z sigmoid(z) sits where 1 + z (1 - sigmoid z) = 0, i.e.
    # sigmoid(z*) = 1 + 1/z*, so its value is v* = z* + 1 (z* about
    # -1.27846).  The grid gives v* to O(h^2); z* = v* - 1 must then hit it.
    zs = np.linspace(-1.4, -1.15, 25001)
    v = np.array([oracle_mod.silu(z) for z in zs])
    i = int(np.argmin(v))
    assert 0 < i < zs.size - 1
    z_star = v[i] - 1.0
    assert abs(z_star + 1.2784645) < 2e-6
    assert abs(oracle_mod.silu(z_star) - v[i]) < 1e-9


def test_epilogue_exact_small_values(oracle_mod):
    t0 = np.array([1.0, 2.0, 3.0, -4.0])
    b0 = np.array([0.5, 0.25, -1.0, 0.0], np.float32)
    r = np.array([0.0, -2.0, 8.0, 0.125], np.float32)
    assert np.array_equal(oracle_mod.epilogue(t0), t0)
    assert np.array_equal(oracle_mod.epilogue(t0, bias0=b0), [1.5, 2.25, 2.0, -4.0])
    assert np.array_equal(oracle_mod.epilogue(t0, residual=r), [1.0, 0.0, 11.0, -3.875])
    assert np.array_equal(oracle_mod.epilogue(t0, bias0=b0, residual=r), [1.5, 0.25, 10.0, -3.875])


def test_swiglu_epilogue_structure(oracle_mod):
    rng = np.random.default_rng(3)
    g = rng.normal(size=64) * 3
    u = rng.normal(size=64)
    out = oracle_mod.epilogue(g, u, swiglu=True)
    ones = oracle_mod.epilogue(g, np.ones(64), swiglu=True)
    # value 1 gives silu(gate); the gate goes through SiLU, the value does not
    assert np.array_equal(ones, [oracle_mod.silu(z) for z in g])
    # linear in the value (powers of two are exact)
    assert np.array_equal(oracle_mod.epilogue(g, 4 * u, swiglu=True), 4 * out)
    # gate 0 gives 0 whatever the value
    assert np.all(oracle_mod.epilogue(np.zeros(64), u, swiglu=True) == 0)
    # biases act before SiLU / the product: shifting t by b equals adding b
    b0 = np.full(64, 0.5, np.float32)
    b1 = np.full(64, -0.25, np.float32)
    assert np.array_equal(oracle_mod.epilogue(g, u, b0, b1, swiglu=True),
                          oracle_mod.epilogue(g + 0.5, u - 0.25, swiglu=True))
    # the residual is added after the product
    r = np.full(64, 2.0, np.float32)
    assert np.array_equal(oracle_mod.epilogue(g, u, residual=r, swiglu=True), out + 2.0)


def test_swiglu_closed_form_on_constant_codes(oracle_mod):
    # All codes 15 (level +1) with scale 1 and x = 1: every row of gate and
    # up is K; silu(K) = K for K = 64 in fp64, so silu(g) * u = K * K.
    M, K = 3, 64
    codes = np.full((M, K // 2), 0xFF, np.uint8)
    scales = np.full((M, K // 64), 0x3C00, np.uint16)   # fp16 1.0
    x = np.full(K, 0x3F80, np.uint16)                    # bf16 1.0
    g, _ = oracle_mod.gemv(codes, scales, M, K, x)
    assert np.array_equal(g, [64.0] * M)
    out = oracle_mod.epilogue(g, g, swiglu=True)
    assert np.array_equal(out, [4096.0] * M)


# ---------------------------------------------------------------------------
# Packed row gather and the bf16 rounding it uses
# ---------------------------------------------------------------------------

def _bf16_value(bits):
    return Fraction(float((np.array([bits], np.uint32) << np.uint32(16)).view(np.float32)[0]))


def _bf16_brute(v):
    """Nearest bf16 pattern to the double v by bisection over the ordered
    positive finite patterns 0x0000..0x7F7F, exact rational distances, ties
    to the even pattern."""
    x = Fraction(v)
    sign = 0x8000 if v < 0 or (v == 0 and np.signbit(v)) else 0
    a = abs(x)
    lo, hi = 0, 0x7F7F
    if a >= _bf16_value(hi):
        lo = hi
    else:
        while hi - lo > 1:  # invariant: value(lo) <= a < value(hi)
            mid = (lo + hi) // 2
            if _bf16_value(mid) <= a:
                lo = mid
            else:
                hi = mid
    if _bf16_value(lo) == a or lo == 0x7F7F and a >= _bf16_value(lo):
        best = lo
    else:
        dl, dh = a - _bf16_value(lo), _bf16_value(hi) - a
        best = lo if dl < dh else hi if dh < dl else (lo if lo % 2 == 0 else hi)
    return sign | best


def test_f64_to_bf16_brute_force(oracle_mod):
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(300) * np.exp2(rng.integers(-30, 30, 300)))
    # exact ties, one ulp either side of them, and the subnormal range
    for m in (1, 3, 5, 127, 255):
        for e in (-20, 0, 7):
            t = (1 + (2 * m - 1) * 2.0 ** -8) * 2.0 ** e if m < 128 else (1 + m * 2.0 ** -8) * 2.0 ** e
            vals += [t, -t, np.nextafter(t, 0), np.nextafter(t, np.inf)]
    vals += [2.0 ** -130, 3 * 2.0 ** -134, 2.0 ** -133 * 1.5, 65504.0, -0.0, 0.0]
    for v in vals:
        assert oracle_mod.f64_to_bf16_bits(v) == _bf16_brute(v), v


def _gather_inputs(oracle_mod, M, K, seed):
    W = wl.weights(M, K, seed, std=0.5)
    codes, scales, st = oracle_mod.pack(W)
    assert st == 0
    return codes, scales


def test_gather_fp32_is_numpy_cast_of_dequant(oracle_mod):
    M, K = 37, 192
    codes, scales = _gather_inputs(oracle_mod, M, K, 11)
    ids = np.array([5, 0, 36, 5, 17, 2], np.int32)
    out, flags = oracle_mod.gather_rows(codes, scales, M, K, ids)
    assert flags == 0
    What = oracle_mod.dequant(codes, scales, M, K)
    assert np.array_equal(out, What[ids].astype(np.float32))


def test_gather_bf16_brute_force(oracle_mod):
    M, K = 9, 128
    codes, scales = _gather_inputs(oracle_mod, M, K, 12)
    ids = np.array([8, 3, 3, 0], np.int32)
    out, flags = oracle_mod.gather_rows(codes, scales, M, K, ids, bf16=True)
    assert flags == 0
    What = oracle_mod.dequant(codes, scales, M, K)
    for i, m in enumerate(ids):
        for k in range(0, K, 3):
            assert out[i, k] == _bf16_brute(What[m, k]), (i, k)


def test_gather_ties_closed_form(oracle_mod):
    """Rows whose blocks hold +s, -s and 0 pack to codes 15, 0, 7 with scale s
    exactly, so the gathered values are +-s and 0: fp32 exact, bf16 the
    nearest-even rounding of s, which for these s is an exact tie."""
    K = 64
    cases = {1 + 2.0 ** -8: 0x3F80, 1 + 3 * 2.0 ** -8: 0x3F82, 2 + 2.0 ** -7: 0x4000,
             0.5 + 3 * 2.0 ** -9: 0x3F02}
    W = np.zeros((len(cases), K), np.float32)
    for r, s in enumerate(cases):
        W[r, 0::3] = s
        W[r, 1::3] = -s
    codes, scales, st = oracle_mod.pack(W)
    assert st == 0
    ids = np.arange(len(cases), dtype=np.int32)
    f32, _ = oracle_mod.gather_rows(codes, scales, len(cases), K, ids)
    b16, _ = oracle_mod.gather_rows(codes, scales, len(cases), K, ids, bf16=True)
    for r, (s, bits) in enumerate(cases.items()):
        assert np.all(f32[r, 0::3] == np.float32(s)) and np.all(f32[r, 1::3] == -np.float32(s))
        assert np.all(f32[r, 2::3] == 0.0)
        assert np.all(b16[r, 0::3] == bits) and np.all(b16[r, 1::3] == (bits | 0x8000))
        assert np.all(b16[r, 2::3] == 0)


def test_gather_refuses_out_of_range_ids(oracle_mod):
    M, K = 6, 64
    codes, scales = _gather_inputs(oracle_mod, M, K, 13)
    ids = np.array([-1, M, 2, 2**31 - 1, 0], np.int32)
    out, flags = oracle_mod.gather_rows(codes, scales, M, K, ids)
    assert flags == oracle_mod.GATHER_BAD_ID
    # accel/tensor func GatherRows: the row of an out-of-range id is zeros
    assert np.all(out[[0, 1, 3]].view(np.uint32) == 0)
    What = oracle_mod.dequant(codes, scales, M, K)
    assert np.array_equal(out[2], What[2].astype(np.float32))
    assert np.array_equal(out[4], What[0].astype(np.float32))
    ok, flags = oracle_mod.gather_rows(codes, scales, M, K, np.array([], np.int32))
    assert flags == 0 and ok.shape == (0, K)


# ---------------------------------------------------------------------------
# Affine 4-bit format: What = (code - z) * s per 64-block
# ---------------------------------------------------------------------------

def test_f64_to_f16_matches_numpy_single_rounding(oracle_mod):
    rng = np.random.default_rng(21)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-30, 17, 3000)))
    # just beyond fp16 ties, where a detour through fp32 would round wrongly
    vals += [1 + 2.0 ** -11 + 2.0 ** -40, 1 + 2.0 ** -11 - 2.0 ** -40, 3 * 2.0 ** -25 + 2.0 ** -60,
             65519.99, 65520.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11]
    for v in vals:
        with np.errstate(over="ignore"):
            ref = int(np.array([np.float16(v)]).view(np.uint16)[0])
        assert oracle_mod.f64_to_f16_bits(v) == ref, v


def _affine_block_params(w):
    """(s, z) of one block from the reading, written independently with exact
    rationals: range widened to hold 0, s = fp16 RNE of range/15 (numpy's
    single rounding of the fp64 quotient), z = nearest integer to -lo/s in
    0..15 with a midpoint going down."""
    lo = min(0.0, float(np.min(w)))
    hi = max(0.0, float(np.max(w)))
    s = float(np.float16((hi - lo) / 15.0))
    if s == 0.0:
        return 0.0, 0
    t = Fraction(-lo) / Fraction(s)
    z = int(t)  # floor (t >= 0)
    if t - z > Fraction(1, 2):
        z += 1
    return s, min(z, 15)


def _affine_unpack(codes, M, K):
    c = np.zeros((M, K), np.int64)
    c[:, 0::2] = codes & 0xF
    c[:, 1::2] = codes >> 4
    return c


def test_affine_pack_brute_force(oracle_mod):
    M, K = 6, 256
    W = wl.weights(M, K, 31, std=0.7)
    W[1, 64:128] += 3.0          # a block far from zero (z = 0 side)
    W[2, 0:64] -= 2.0            # and the other side (z = 15)
    W[3, 128:192] = 0.0          # all zero: s = 0
    W[4, 192:256] = 0.25         # constant positive
    codes, scales, zeros, st = oracle_mod.pack_affine(W)
    assert st == 0
    c = _affine_unpack(codes, M, K)
    for m in range(M):
        for b in range(K // 64):
            w = W[m, 64 * b:64 * b + 64].astype(np.float64)
            s, z = _affine_block_params(w)
            assert scales[m, b] == np.array([np.float16(s)]).view(np.uint16)[0]
            assert zeros[m, b] == np.array([np.float16(z)]).view(np.uint16)[0]
            lv = (np.arange(16) - z) * s
            for k in range(64):
                code = c[m, 64 * b + k]
                if s == 0.0:
                    assert code == 0
                    continue
                d = np.abs(lv - w[k])
                best = int(np.flatnonzero(d == d.min())[0])  # lowest code on a tie
                assert code == best, (m, b, k)


def test_affine_closed_forms(oracle_mod):
    K = 64
    W = np.zeros((4, K), np.float32)
    W[0, :] = 0.25                       # [0, 0.25]: z = 0, codes 15
    W[1, :] = -1.5                       # [-1.5, 0]: s = 0.1, z = 15, codes 0
    W[2, 0::2], W[2, 1::2] = 1.5, -1.5   # [-1.5, 1.5]: s = 0.2, z = 7.5 -> 7 (midpoint down)
    codes, scales, zeros, st = oracle_mod.pack_affine(W)
    assert st == 0
    s = scales.view(np.float16).astype(np.float64)
    z = zeros.view(np.float16).astype(np.float64)
    c = _affine_unpack(codes, 4, K)
    assert s[0, 0] == np.float16(0.25 / 15) and z[0, 0] == 0 and np.all(c[0] == 15)
    assert s[1, 0] == np.float16(0.1) and z[1, 0] == 15 and np.all(c[1] == 0)
    assert s[2, 0] == np.float16(0.2)
    assert z[2, 0] == (7 if 1.5 / float(np.float16(0.2)) <= 7.5 else 8)  # fp16(0.2) < 0.2: 8
    assert np.all(s[3] == 0) and np.all(z[3] == 0) and np.all(c[3] == 0)
    What = oracle_mod.dequant_affine(codes, scales, zeros, 4, K)
    assert np.all(What[3] == 0.0)
    assert np.all(What[0] == 15 * s[0, 0]) and np.all(What[1] == -15 * s[1, 0])


def test_affine_error_is_at_most_range_over_30(oracle_mod):
    M, K = 64, 512
    W = wl.weights(M, K, 32, std=1.0) + np.float32(0.3)
    codes, scales, zeros, st = oracle_mod.pack_affine(W)
    assert st == 0
    What = oracle_mod.dequant_affine(codes, scales, zeros, M, K)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 64, axis=1)
    err = np.abs(What - W)
    # half a level step, plus the fp16 rounding of s stretched over 15 steps
    assert np.all(err <= s * (0.5 + 15 * 2.0 ** -11) + 1e-12)
    blk = W.reshape(M, K // 64, 64).astype(np.float64)
    rng_ = np.maximum(blk.max(2), 0) - np.minimum(blk.min(2), 0)
    assert np.all(err.reshape(M, K // 64, 64).max(2) <= rng_ / 30 * (1 + 2.0 ** -9) + 1e-12)


def test_affine_refuses_nonfinite_and_overflow(oracle_mod):
    W = np.zeros((3, 128), np.float32)
    W[0, 3] = np.nan
    W[1, 70] = np.inf
    _, _, _, st = oracle_mod.pack_affine(W[:2])
    assert st == oracle_mod.PACK_NONFINITE
    W2 = np.zeros((1, 64), np.float32)
    W2[0, 0], W2[0, 1] = 6.0e5, -6.0e5  # range / 15 = 8e4 >= 65520
    assert oracle_mod.pack_affine(W2)[3] == oracle_mod.PACK_OVERFLOW
    W2[0, 0], W2[0, 1] = 4.0e5, -4.0e5  # 53333: fits
    assert oracle_mod.pack_affine(W2)[3] == 0


def test_affine_dequant_hand_built(oracle_mod):
    K = 64
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 0] = 0x5A  # k=0 -> code 10, k=1 -> code 5
    codes[0, 1] = 0xF0  # k=2 -> 0, k=3 -> 15
    scales = np.array([[np.float16(0.5)]]).view(np.uint16)
    zeros = np.array([[np.float16(6.0)]]).view(np.uint16)
    What = oracle_mod.dequant_affine(codes, scales, zeros, 1, K)
    assert list(What[0, :4]) == [2.0, -0.5, -3.0, 4.5]
    assert np.all(What[0, 4:] == -3.0)


def test_affine_gemv_matches_blas_and_one_hot(oracle_mod):
    M, K = 33, 320
    W = wl.weights(M, K, 33, std=0.5)
    codes, scales, zeros, st = oracle_mod.pack_affine(W)
    x = wl.activation(K, 33, "normal")
    y, S = oracle_mod.gemv_affine(codes, scales, zeros, M, K, x)
    What = oracle_mod.dequant_affine(codes, scales, zeros, M, K)
    xv = wl.bf16_bits_to_f32(x).astype(np.float64)
    assert np.allclose(y, What @ xv, rtol=1e-12, atol=1e-12)
    assert np.allclose(S, np.abs(What) @ np.abs(xv), rtol=1e-12)
    for k in (0, 63, 64, 319):
        e = np.zeros(K, np.uint16)
        e[k] = 0x3F80  # bf16 1.0
        yk, _ = oracle_mod.gemv_affine(codes, scales, zeros, M, K, e)
        assert np.array_equal(yk, What[:, k])


def test_affine_gemm_matches_blas(oracle_mod):
    """The prefill product of the affine format against a BLAS product of
    the dequantised matrix (an independent path: the matrix is built by
    oracle_dequant_affine, the product by numpy)."""
    M, K, N = 40, 320, 5
    W = wl.weights(M, K, 61)
    X = wl.activations(N, K, 61, "unit_rms")
    codes, scales, zeros, st = oracle_mod.pack_affine(W)
    assert st == 0
    Y, S = oracle_mod.gemm_affine(codes, scales, zeros, M, K, X)
    What = oracle_mod.dequant_affine(codes, scales, zeros, M, K)
    Xv = wl.bf16_bits_to_f32(X).astype(np.float64)
    assert np.all(np.abs(Y - Xv @ What.T) <= 1e-12 * (np.abs(Xv) @ np.abs(What).T))
    assert np.allclose(S, np.abs(Xv) @ np.abs(What).T, rtol=1e-12, atol=0)


def test_affine_exact_ties_go_down(oracle_mod):
    """s = 0.125 exactly (range 1.875 / 15) and -lo / s = 7.5 exactly: z takes
    the lower integer 7; weights on a level midpoint take the lower code."""
    W = np.zeros((1, 64), np.float32)
    W[0, :4] = [0.9375, -0.9375, 0.0625, -0.0625]
    W[0, 4] = 0.1875  # midpoint of levels 1*s and 2*s above z
    codes, scales, zeros, st = oracle_mod.pack_affine(W)
    assert st == 0
    assert scales.view(np.float16)[0, 0] == 0.125 and zeros.view(np.float16)[0, 0] == 7.0
    c = _affine_unpack(codes, 1, 64)
    assert list(c[0, :5]) == [14, 0, 7, 6, 8]
    What = oracle_mod.dequant_affine(codes, scales, zeros, 1, 64)
    assert list(What[0, :5]) == [0.875, -0.875, 0.0, -0.125, 0.125]


# ---------------------------------------------------------------------------
# NVFP4-style format: E2M1 codes, E4M3 scale per 16 along K, f32 tensor scale
# ---------------------------------------------------------------------------

def _e4m3_exact(b):
    """E4M3FN from its definition (bias 7, subnormals (m/8) 2^-6, 0x7F NaN)."""
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return None
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


_E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
_E4M3_POS = [_e4m3_exact(b) for b in range(127)]


def test_e4m3_and_e2m1_values(oracle_mod):
    import torch
    tv = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for b in range(256):
        v = oracle_mod.e4m3_to_f64(b)
        ref = _e4m3_exact(b)
        if ref is None:
            assert np.isnan(v) and np.isnan(tv[b])
        else:
            assert Fraction(v) == ref and v == tv[b], b
    # E2M1 from its definition: bias 1, e = 0 -> m / 2, else 2^(e-1) (1 + m/2)
    for c in range(16):
        e, m = (c >> 1) & 3, c & 1
        mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
        assert Fraction(oracle_mod.e2m1_to_f64(c)) == (-mag if c & 8 else mag), c


def _nearest_even(a, grid):
    """Index of the grid value nearest to the rational a >= 0, ties to the even
    index, saturating at the top."""
    best = None
    for i, g in enumerate(grid):
        d = abs(a - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def test_nvfp4_pack_brute_force(oracle_mod):
    M, K = 5, 128
    W = wl.weights(M, K, 41, std=0.5)
    W[1, 16:32] *= 1e-4                 # a small block (subnormal E4M3 scale)
    W[2, 32:48] = 0.0                   # a zero block
    W[3, 0] = -0.0
    codes, scales, s, st = oracle_mod.pack_nvfp4(W)
    assert st == 0
    assert s == np.float32(np.max(np.abs(W)).astype(np.float64) / 2688.0)
    S = Fraction(float(s))
    for m in range(M):
        for b in range(K // 16):
            w = W[m, 16 * b:16 * b + 16]
            amax = Fraction(float(np.max(np.abs(w))))
            sb = _nearest_even(amax / (6 * S), _E4M3_POS)
            assert scales[m, b] == sb, (m, b)
            unit = _E4M3_POS[sb] * S
            for k in range(16):
                byte = codes[m, 8 * b + k // 2]
                c = (byte >> 4) if k % 2 else (byte & 15)
                wk = float(w[k])
                if unit == 0:
                    assert c == 0
                    continue
                mag = _nearest_even(abs(Fraction(wk)) / unit, _E2M1)
                assert c == (mag | (8 if np.signbit(wk) else 0)), (m, b, k)


def test_nvfp4_closed_forms_and_ties(oracle_mod):
    """max |W| = 2688 makes s = 1; a block with amax 6 gets scale 1.0 (0x38)
    and values on the E2M1 grid and on its midpoints (ties to the even code);
    amax 6.375 = 6 * 1.0625 is the midpoint of E4M3 1.0 and 1.125: scale 1.0,
    and 6.375 itself saturates to 6."""
    W = np.zeros((1, 64), np.float32)
    W[0, 0] = 2688.0
    W[0, 16:32] = [6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -5, 0.5, 3, 0, -6, 4, 1.5]
    W[0, 32:34] = [6.375, 1.0]
    codes, scales, s, st = oracle_mod.pack_nvfp4(W)
    assert st == 0 and s == 1.0
    assert scales[0, 0] == 0x7E  # 2688 / 6 = 448
    assert scales[0, 1] == 0x38 and scales[0, 2] == 0x38
    c = np.zeros(64, np.int64)
    c[0::2], c[1::2] = codes[0] & 15, codes[0] >> 4
    assert list(c[16:32]) == [7, 0, 2, 2, 4, 4, 6, 6, 8, 14, 1, 5, 0, 15, 6, 3]
    assert list(c[32:34]) == [7, 2]
    What = oracle_mod.dequant_nvfp4(codes, scales, s, 1, 64)
    assert What[0, 32] == 6.0 and What[0, 0] == 2688.0


def test_nvfp4_gemm_matches_blas(oracle_mod):
    """The NVFP4-style prefill product against a BLAS product of the
    dequantised matrix."""
    M, K, N = 40, 320, 5
    W = wl.weights(M, K, 62)
    X = wl.activations(N, K, 62, "swiglu")
    codes, scales, s, st = oracle_mod.pack_nvfp4(W)
    assert st == 0
    Y, S = oracle_mod.gemm_nvfp4(codes, scales, s, M, K, X)
    What = oracle_mod.dequant_nvfp4(codes, scales, s, M, K)
    Xv = wl.bf16_bits_to_f32(X).astype(np.float64)
    assert np.all(np.abs(Y - Xv @ What.T) <= 1e-12 * (np.abs(Xv) @ np.abs(What).T))
    assert np.allclose(S, np.abs(Xv) @ np.abs(What).T, rtol=1e-12, atol=0)


def test_nvfp4_zero_tensor_and_refusal(oracle_mod):
    W = np.zeros((2, 64), np.float32)
    codes, scales, s, st = oracle_mod.pack_nvfp4(W)
    assert st == 0 and s == 0.0 and not codes.any() and not scales.any()
    W[1, 5] = np.inf
    assert oracle_mod.pack_nvfp4(W)[3] == oracle_mod.PACK_NONFINITE


def test_nvfp4_gemv_matches_blas_and_one_hot(oracle_mod):
    M, K = 21, 192
    W = wl.weights(M, K, 43, std=0.5)
    codes, scales, s, st = oracle_mod.pack_nvfp4(W)
    x = wl.activation(K, 43, "normal")
    y, S = oracle_mod.gemv_nvfp4(codes, scales, s, M, K, x)
    What = oracle_mod.dequant_nvfp4(codes, scales, s, M, K)
    xv = wl.bf16_bits_to_f32(x).astype(np.float64)
    assert np.allclose(y, What @ xv, rtol=1e-12, atol=1e-12)
    assert np.allclose(S, np.abs(What) @ np.abs(xv), rtol=1e-12)
    for k in (0, 15, 16, 191):
        e = np.zeros(K, np.uint16)
        e[k] = 0x3F80
        yk, _ = oracle_mod.gemv_nvfp4(codes, scales, s, M, K, e)
        assert np.array_equal(yk, What[:, k])
    # a hand-built element: code 0xB (-1.5) with scale 0x30 (0.5) and s
    cb = np.zeros((1, 32), np.uint8)
    cb[0, 0] = 0xB0  # k=0 code 0, k=1 code 0xB
    sc = np.full((1, 4), 0x30, np.uint8)
    Wh = oracle_mod.dequant_nvfp4(cb, sc, np.float32(0.25), 1, 64)
    assert Wh[0, 0] == 0.0 and Wh[0, 1] == -1.5 * 0.5 * 0.25


# ---------------------------------------------------------------------------
# int8 activations (one or two words) and the affine GEMV on them
# ---------------------------------------------------------------------------

def _nearest_int_even(t):
    """Nearest integer to the rational t >= 0, ties to even, at most 127."""
    j = int(t)
    f = t - j
    if f > Fraction(1, 2) or (f == Fraction(1, 2) and j % 2 == 1):
        j += 1
    return min(j, 127)


def _bf16_from_values(vals):
    b = np.array(vals, np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "fixture values must be bf16"
    return (b >> 16).astype(np.uint16)


def test_quantize_x8_brute_force(oracle_mod):
    x = wl.activation(256, 51, "normal")
    x[40] = 0x8000  # -0.0
    for words in (1, 2):
        q1, q2, d = oracle_mod.quantize_x8(x, words)
        xv = wl.bf16_bits_to_f32(x).astype(np.float64)
        for b in range(8):
            blk = xv[32 * b:32 * b + 32]
            assert d[b] == np.float32(np.max(np.abs(blk)) / 127.0)
            D = Fraction(float(d[b]))
            for k in range(32):
                v = Fraction(float(blk[k]))
                a1 = _nearest_int_even(abs(v) / D) * (1 if v >= 0 else -1)
                assert q1[32 * b + k] == a1
                if words == 2:
                    r = v - a1 * D
                    a2 = _nearest_int_even(abs(r) * 128 / D) * (1 if r >= 0 else -1)
                    assert q2[32 * b + k] == a2


def test_quantize_x8_ties_and_bounds(oracle_mod):
    vals = np.zeros(32, np.float32)
    vals[:6] = [127.0, 2.5, 3.5, -2.5, 0.5, 0.50390625]  # d = 1: ties to 2, 4, -2, 0, and 1 + (-63.5 -> -64)/128
    x = _bf16_from_values(vals)
    q1, q2, d = oracle_mod.quantize_x8(x, 2)
    assert d[0] == 1.0
    assert list(q1[:6]) == [127, 2, 4, -2, 0, 1]
    assert q2[5] == -64 and q2[4] == 64
    # the bounds |x - xq| <= d/2 (one word) and d/256 (two words)
    xr = wl.activation(4096, 52, "normal")
    xv = wl.bf16_bits_to_f32(xr).astype(np.float64)
    for words, lim in ((1, 0.5), (2, 1.0 / 256)):
        a, b2, dd = oracle_mod.quantize_x8(xr, words)
        xq = oracle_mod.dequantize_x8(a, b2, dd)
        assert np.all(np.abs(xq - xv) <= lim * np.repeat(dd.astype(np.float64), 32))
    z = np.zeros(64, np.uint16)
    a, b2, dd = oracle_mod.quantize_x8(z, 2)
    assert not a.any() and not b2.any() and not dd.any()


def test_affine_x8_gemv_matches_blas_and_exact_case(oracle_mod):
    M, K = 19, 256
    W = wl.weights(M, K, 53, std=0.5)
    codes, scales, zeros, st = oracle_mod.pack_affine(W)
    x = wl.activation(K, 53, "normal")
    for words in (1, 2):
        q1, q2, d = oracle_mod.quantize_x8(x, words)
        y, S = oracle_mod.gemv_affine_x8(codes, scales, zeros, M, K, q1, q2, d)
        What = oracle_mod.dequant_affine(codes, scales, zeros, M, K)
        xq = oracle_mod.dequantize_x8(q1, q2, d)
        assert np.allclose(y, What @ xq, rtol=1e-12, atol=1e-12)
        assert np.allclose(S, np.abs(What) @ np.abs(xq), rtol=1e-12)
    # integer activations with each block's maximum 127: d = 1, xq == x, so
    # the product equals the bf16 GEMV bit for bit
    rng = np.random.default_rng(54)
    iv = rng.integers(-127, 128, K).astype(np.float32)
    iv[::32] = 127.0
    xi = _bf16_from_values(iv)
    q1, q2, d = oracle_mod.quantize_x8(xi, 2)
    assert np.all(d == 1.0) and not q2.any()
    y8, _ = oracle_mod.gemv_affine_x8(codes, scales, zeros, M, K, q1, q2, d)
    yb, _ = oracle_mod.gemv_affine(codes, scales, zeros, M, K, xi)
    assert np.array_equal(y8, yb)
