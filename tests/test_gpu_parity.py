"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Acceptance (the bar of this library):
  - q4_pack: codes and scale bits equal, bit for bit;
  - q4_gemv / q4_gemm_smalln: |y - y_ref| <= 1e-3 * sum_k |What x| + 1e-5 per output;
  - lm_head-shaped outputs: identical argmax (ties to the lowest index,
    golang.design accel/tensor func Argmax).
Inputs come from the seeded generators; the oracle never sees anything the
GPU produced.  Without a GPU these tests SKIP; they never pass silently.
"""
import os
import sys
import time

import numpy as np
import pytest

import cases
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


def _log(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible: SKIP (not a pass)")
    import bit_weight_gemv_amd as q4
    q4.lib()  # raises if libq4.so is missing: no fallback exists
    oracle.build(force=False)
    return torch, q4, torch.device("cuda:0")


def _gpu_pack(env, W):
    torch, q4, dev = env
    Wd = cases.to_dev(W, torch, dev)
    codes, scales, status = q4.q4_pack(Wd)
    torch.cuda.synchronize()
    return codes, scales, int(status.item())


def _upload_packed(env, codes, scales):
    torch, q4, dev = env
    c = cases.to_dev(codes, torch, dev)
    s = cases.to_dev(scales.view(np.float16), torch, dev)
    return c, s


def _x_dev(env, x_bits):
    torch, q4, dev = env
    return cases.to_dev(x_bits.view(np.int16), torch, dev).view(torch.bfloat16)


def _check(y_gpu, y_ref, S, what):
    ok, ratio = oracle.within_tolerance(y_gpu, y_ref, S)
    _log(f"{what}: worst |err|/bound = {ratio:.3g}")
    assert ok, f"{what}: tolerance broken, worst ratio {ratio}"


# ---------------------------------------------------------------------------
# q4_pack
# ---------------------------------------------------------------------------

PACK_SHAPES = [(1, 64), (3, 128), (17, 192), (256, 512), (5, 4096), (33, 11008)]


@pytest.mark.parametrize("M,K", PACK_SHAPES)
def test_pack_bit_exact_random(env, M, K):
    W = wl.weights(M, K, seed=100 + M + K)
    c_ref, s_ref, st_ref = oracle.pack(W)
    codes, scales, st = _gpu_pack(env, W)
    assert st == st_ref == 0
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(cases.bits16(scales, env[0]), s_ref)


@pytest.mark.parametrize("M,K", [(3, 128), (257, 512), (33, 11008)])
def test_unpack_canonical_bit_exact(env, M, K):
    torch, q4, dev = env
    W = wl.weights(M, K, seed=700 + M + K)
    c_ref, s_ref, _ = oracle.pack(W)
    codes, scales, st = _gpu_pack(env, W)
    assert st == 0
    co, so = q4.q4_unpack_canonical(codes, scales)
    torch.cuda.synchronize()
    assert np.array_equal(co.cpu().numpy(), c_ref)
    assert np.array_equal(cases.bits16(so, torch), s_ref)
    assert co.data_ptr() != codes.data_ptr() and so.data_ptr() != scales.data_ptr()


def test_pack_bit_exact_edge_blocks(env):
    W = cases.edge_matrix()
    c_ref, s_ref, st_ref = oracle.pack(W)
    codes, scales, st = _gpu_pack(env, W)
    assert st == st_ref == 0
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(cases.bits16(scales, env[0]), s_ref)


def test_pack_bit_exact_scaled_range(env):
    # the same weights at many magnitudes, including fp16-subnormal scales
    base = wl.weights(40, 256, seed=7)
    W = np.concatenate([base * np.float32(2.0 ** j) for j in range(-30, 16, 3)]).astype(np.float32)
    c_ref, s_ref, st_ref = oracle.pack(W)
    codes, scales, st = _gpu_pack(env, W)
    assert st == st_ref == 0
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(cases.bits16(scales, env[0]), s_ref)


def test_pack_flags_and_valid_blocks(env):
    W = wl.weights(8, 256, seed=3)
    W[1, 70] = np.nan
    W[2, 3] = np.inf
    W[5, 200] = -70000.0
    c_ref, s_ref, st_ref = oracle.pack(W)
    codes, scales, st = _gpu_pack(env, W)
    assert st == st_ref == (oracle.PACK_NONFINITE | oracle.PACK_OVERFLOW)
    codes = codes.cpu().numpy()
    scales = cases.bits16(scales, env[0])
    good = np.ones((8, 4), bool)
    good[1, 1] = good[2, 0] = good[5, 3] = False
    for m in range(8):
        for b in range(4):
            if good[m, b]:
                assert np.array_equal(codes[m, 32 * b:32 * b + 32], c_ref[m, 32 * b:32 * b + 32])
                assert scales[m, b] == s_ref[m, b]
    # a second clean call clears the word
    _, _, st2 = _gpu_pack(env, wl.weights(8, 256, seed=3))
    assert st2 == 0


# ---------------------------------------------------------------------------
# q4_gemv
# ---------------------------------------------------------------------------

# (M, K): several tiles and ragged tails for every launch shape:
#   K <= 2048: a wave per row, one 4-row tile per wave up to 16 tiles per CU
#     (16384 rows with 256 CUs), tiles dealt to the waves in turn beyond;
#   K <= 32768: a group of waves per row tile, one chunk a lane;
#   longer rows: 4 chunks a lane (K <= 65536), else 8.
GEMV_SHAPES = [(1, 64), (2, 64), (7, 128), (257, 512), (1000, 1024), (4097, 2048), (31, 1984),
               (32771, 192), (40001, 64),
               (300, 2112), (65, 4096), (129, 4160), (2048, 11008), (33, 11008), (9, 16384),
               (4099, 4160), (5, 16448), (4101, 16448), (3, 32768), (2, 65536), (2, 131072),
               # long rows in two workgroups per CU, several groups each, some
               # groups one tile short of the others
               (8197, 6208),
               # rows of one wave dealt to the waves in turn (more than 16
               # tiles per CU), with ragged last tiles
               (16389, 1024), (20011, 2048)]


@pytest.mark.parametrize("M,K", GEMV_SHAPES)
def test_gemv_parity_shapes(env, M, K):
    torch, q4, dev = env
    seed = 1000 + M + K
    W = wl.weights(M, K, seed)
    x = wl.activation(K, seed, "normal")
    codes, scales, st = oracle.pack(W)
    assert st == 0
    y_ref, S = oracle.gemv(codes, scales, M, K, x)
    c, s = _upload_packed(env, codes, scales)
    y = q4.q4_gemv(c, s, _x_dev(env, x))
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), y_ref, S, f"gemv M={M} K={K}")


def _scales_at(env, scales, shift):
    """The scales on the device at a 2-byte offset of `shift` units from a
    fresh (256-byte aligned) allocation: shift 1 leaves the plane 2 mod 4."""
    torch, q4, dev = env
    buf = torch.zeros(scales.size + shift, dtype=torch.float16, device=dev)
    buf[shift:].copy_(torch.from_numpy(scales.reshape(-1).view(np.float16)))
    return buf[shift:].view(scales.shape)


# (M, K) with odd and even scale counts per row (K / 64), in the row ranges of
# one tile per wave (at most 4096 four-row tiles), in the strided order
# (more) and in rows spanning several waves: with one chunk a lane the
# GEMV reads a tile's scales with one dword load per lane
# (handed on by quad broadcasts) when the plane is dword-aligned and a row
# holds an even number of scales, else one 2-byte load per row; both are
# checked on a dword-aligned and on a 2 mod 4 scale plane.
SCALE_RUN_SHAPES = [(37, 64), (1001, 192), (257, 576), (130, 1984), (1001, 128), (300, 1024), (129, 2048),
                    (16411, 64), (17003, 576), (16389, 1984), (20011, 2048),
                    # rows spanning several waves (one chunk a lane)
                    (2053, 11008), (517, 5120), (1001, 4224), (33, 6208), (3001, 2112)]


@pytest.mark.parametrize("shift", [0, 1])
@pytest.mark.parametrize("M,K", SCALE_RUN_SHAPES)
def test_gemv_scale_runs_every_alignment(env, M, K, shift):
    torch, q4, dev = env
    seed = 2000 + M + K
    W = wl.weights(M, K, seed)
    x = wl.activation(K, seed, "unit_rms")
    codes, scales, st = oracle.pack(W)
    assert st == 0
    y_ref, S = oracle.gemv(codes, scales, M, K, x)
    c, _ = _upload_packed(env, codes, scales)
    s = _scales_at(env, scales, shift)
    assert s.data_ptr() % 4 == 2 * shift
    y = q4.q4_gemv(c, s, _x_dev(env, x))
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), y_ref, S, f"gemv M={M} K={K} scale plane +{2 * shift} B")


# SwiGLU pairs as the halves of one packed matrix: with an odd number of
# scales per row and an odd M the up half's plane is 2 mod 4.
@pytest.mark.parametrize("M,K", [(1101, 576), (1100, 576), (1100, 1024), (9001, 192), (9000, 192), (9000, 2048)])
def test_fused_swiglu_scale_plane_alignment(env, M, K):
    torch, q4, dev = env
    W = wl.weights(2 * M, K, 6500 + M)
    x = wl.activation(K, 6500 + M, "unit_rms")
    codes, scales, _ = oracle.pack(W)
    t, S = oracle.gemv(codes, scales, 2 * M, K, x)
    c, s = _upload_packed(env, codes, scales)
    _log(f"swiglu M={M} K={K}: up scales at {s[M:].data_ptr() % 4} mod 4")
    ops = [(c[:M], s[:M], None), (c[M:], s[M:], None)]
    y = q4.q4_gemv_fused(ops, _x_dev(env, x), "swiglu")[0]
    torch.cuda.synchronize()
    y_ref, bound = _fused_ref([t[:M], t[M:]], [S[:M], S[M:]], [None, None], [None], True)
    _check_bound(y.cpu().numpy(), y_ref[0], bound[0], f"swiglu halves M={M} K={K}")


def test_gemv_after_gpu_pack_matches_oracle_chain(env):
    torch, q4, dev = env
    M, K = 700, 2048
    W = wl.weights(M, K, 5)
    x = wl.activation(K, 5, "unit_rms")
    c_ref, s_ref, _ = oracle.pack(W)
    y_ref, S = oracle.gemv(c_ref, s_ref, M, K, x)
    codes, scales, st = _gpu_pack(env, W)
    y = q4.q4_gemv(codes, scales, _x_dev(env, x))
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), y_ref, S, "pack+gemv")


def _bf16_bits(v):
    return wl.bf16_rne_bits(np.asarray(v, np.float64))


@pytest.mark.parametrize("kind", ["huge", "tiny", "mixed", "zeros", "onehot", "fp16_edge"])
def test_gemv_activation_ranges(env, kind):
    torch, q4, dev = env
    M, K = 130, 2048
    W = wl.weights(M, K, 9)
    codes, scales, _ = oracle.pack(W)
    rng = np.random.default_rng(4)
    z = rng.standard_normal(K)
    if kind == "huge":
        v = z * 1e30
    elif kind == "tiny":
        v = z * 1e-30
    elif kind == "mixed":
        v = z * np.exp2(rng.integers(-60, 60, K))
    elif kind == "zeros":
        v = np.zeros(K)
    elif kind == "onehot":
        v = np.zeros(K)
        v[777] = 1.0
    else:  # values just above fp16 range and around its subnormals
        v = np.where(rng.random(K) < 0.5, 70000.0, 3e-6) * np.sign(z)
    x = _bf16_bits(v)
    y_ref, S = oracle.gemv(codes, scales, M, K, x)
    c, s = _upload_packed(env, codes, scales)
    y = q4.q4_gemv(c, s, _x_dev(env, x))
    torch.cuda.synchronize()
    yg = y.cpu().numpy()
    if kind in ("zeros",):
        assert np.all(yg == 0)
    _check(yg, y_ref, S, f"gemv x={kind}")


# ---------------------------------------------------------------------------
# Activations of any range.  An fp16 copy of a wave's activations under one
# power of two (the integer conversion on the bf16 bits) is exact only while
# they span at most 2^28; beyond that the kernels take the raw bf16 values.
# Each case puts a huge activation where it meets only zero weights (a zero
# 64-block, or a column of code 7), so the row sums come entirely from
# activations far below it: a conversion that flushed them would give y = 0.
# spread_28 / spread_29 sit on the exactness threshold with activations
# 1 + 2^-7 (8 significant bits), which a conversion taken one binade too far
# would turn into wrong fp16 patterns; spread_31 / spread_32 lie past it.
# ---------------------------------------------------------------------------

# spread_n: unit magnitudes and one value 2^n: n = 28 is the widest spread the
# integer conversion holds exactly (fp16 normal numbers).
WIDE_KINDS = ["zero_block_2^60", "code7_column_2^60", "spread_28", "spread_29", "spread_31", "spread_32", "tiny_run",
              "many_windows"]
K_ZERO_BLOCK, K_ZERO_COL = 64 * 3 + 5, 1000


def _wide_x(kind, K, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(K)
    sgn = np.where(z < 0, -1.0, 1.0)
    if kind == "zero_block_2^60":
        v = z.copy()
        v[K_ZERO_BLOCK] = 2.0 ** 60
    elif kind == "code7_column_2^60":
        v = z.copy()
        v[K_ZERO_COL] = -(2.0 ** 60)
    elif kind.startswith("spread_"):
        v = sgn * (1.0 + 2.0 ** -7)
        v[K_ZERO_COL] = 2.0 ** int(kind[-2:])
    elif kind == "tiny_run":
        v = z.copy()
        v[100:140] *= 2.0 ** -100
        v[K_ZERO_COL] = 2.0 ** 50
    else:  # many_windows: magnitudes over 160 binades (five windows), every weight nonzero
        v = sgn * (1.0 + 0.5 * rng.random(K)) * np.exp2(rng.integers(-120, 41, K).astype(np.float64))
    return _bf16_bits(v)


def _wide_w(W):
    W = W.copy()
    b = K_ZERO_BLOCK // 64
    W[:, 64 * b:64 * b + 64] = 0.0
    W[:, K_ZERO_COL] = 0.0
    return W


WIDE_GEMV_SHAPES = [(300, 2048), (20011, 2048), (77, 11008), (64, 4096), (5, 40960), (3, 98304)]


@pytest.mark.parametrize("kind", WIDE_KINDS)
@pytest.mark.parametrize("M,K", WIDE_GEMV_SHAPES)
def test_gemv_wide_range_activations(env, M, K, kind):
    torch, q4, dev = env
    seed = 7300 + M + K
    W = _wide_w(wl.weights(M, K, seed))
    x = _wide_x(kind, K, seed)
    codes, scales, _ = oracle.pack(W)
    y_ref, S = oracle.gemv(codes, scales, M, K, x, threads=min(16, os.cpu_count() or 1))
    c, s = _upload_packed(env, codes, scales)
    y = q4.q4_gemv(c, s, _x_dev(env, x))
    torch.cuda.synchronize()
    yg = y.cpu().numpy()
    assert np.all(np.isfinite(yg))
    _check(yg, y_ref, S, f"gemv wide x={kind} M={M} K={K}")


@pytest.mark.parametrize("kind", WIDE_KINDS)
@pytest.mark.parametrize("M,K", [(300, 2048), (77, 11008)])
def test_affine_and_nvfp4_wide_range_activations(env, M, K, kind):
    torch, q4, dev = env
    seed = 7400 + M + K
    W = _wide_w(wl.weights(M, K, seed, std=0.5))
    x = _wide_x(kind, K, seed)
    codes, scales, zeros, st = oracle.pack_affine(W)
    assert st == 0
    y_ref, S = oracle.gemv_affine(codes, scales, zeros, M, K, x)
    c, s, z = _affine_upload(env, codes, scales, zeros)
    y = q4.q4_gemv_affine(c, s, z, _x_dev(env, x))
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), y_ref, S, f"affine gemv wide x={kind} M={M} K={K}")
    ncodes, nscales, ts, st = oracle.pack_nvfp4(W)
    assert st == 0
    y_ref, S = oracle.gemv_nvfp4(ncodes, nscales, ts, M, K, x)
    t = torch.tensor([ts], dtype=torch.float32, device=dev)
    y = q4.q4_gemv_nvfp4(cases.to_dev(ncodes, torch, dev), cases.to_dev(nscales, torch, dev), t, _x_dev(env, x))
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), y_ref, S, f"nvfp4 gemv wide x={kind} M={M} K={K}")


@pytest.mark.parametrize("M,K,N", [(300, 2048, 2), (300, 2048, 3), (3001, 1984, 3), (600, 11008, 1),
                                   (300, 2048, 4), (300, 2048, 17), (3001, 1984, 32), (77, 4160, 17),
                                   (70, 11008, 32), (300, 2048, 8), (300, 2048, 16), (3001, 1920, 11),
                                   (300, 11008, 2), (77, 4160, 3), (50, 8192, 4)])
def test_gemm_smalln_wide_range_activations(env, M, K, N):
    """Each token of the chunk takes a different wide-range recipe."""
    torch, q4, dev = env
    seed = 7500 + M + K + N
    W = _wide_w(wl.weights(M, K, seed))
    X = np.stack([_wide_x(WIDE_KINDS[(n + seed) % len(WIDE_KINDS)], K, seed + n) for n in range(N)])
    codes, scales, _ = oracle.pack(W)
    Y_ref, S = oracle.gemm(codes, scales, M, K, X)
    c, s = _upload_packed(env, codes, scales)
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    Y = q4.q4_gemm_smalln(c, s, Xd)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"gemm wide M={M} K={K} N={N}")


@pytest.mark.parametrize("kind", ["code7_column_2^60", "spread_32", "many_windows"])
@pytest.mark.parametrize("swiglu,Ms,K", [(False, (2048, 256, 256), 2048), (False, (300, 40), 11008),
                                         (True, (1000, 1000), 2048), (True, (300, 300), 4160)])
def test_fused_wide_range_activations(env, swiglu, Ms, K, kind):
    seed = 7600 + K + sum(Ms)
    # Bias and residual small next to the products, so the products' bound
    # is what is tested.
    _fused_case(env, Ms, K, seed, swiglu=swiglu, x=_wide_x(kind, K, seed), w_hook=_wide_w, bias_scale=1e-3)


# The prefill product of the affine and NVFP4-style formats: one token (the
# format's GEMV), two and three tokens, one and two 16-token halves,
# activations in registers (K <= 2048, ragged last slice) and reloaded per
# tile (longer rows), many tiles per workgroup.  2..8 tokens on rows of at
# most 2048 weights with K % 128 == 0 take the 4-row-tile kernel: one and
# two token groups, ragged last tile and partial last group, rows shorter
# than a load, one tile.
FMT_GEMM_CASES = [(300, 2048, 1), (300, 2048, 2), (1000, 1984, 3), (77, 4160, 17), (300, 2048, 32),
                  (20000, 192, 5), (50, 2112, 20), (70, 11008, 32), (1, 64, 2),
                  (3001, 1920, 4), (13, 640, 7), (12288, 2048, 8), (4099, 1152, 6), (2, 256, 5),
                  (1, 128, 3), (257, 2048, 8), (11008, 2048, 2)]


def _nvfp4_upload(env, codes, scales, ts):
    torch, q4, dev = env
    return (cases.to_dev(codes, torch, dev), cases.to_dev(scales, torch, dev),
            torch.tensor([ts], dtype=torch.float32, device=dev))


def _gemm_formats_case(env, M, K, N, W, X, what):
    torch, q4, dev = env
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    codes, scales, zeros, st = oracle.pack_affine(W)
    assert st == 0
    Y_ref, S = oracle.gemm_affine(codes, scales, zeros, M, K, X)
    c, s, z = _affine_upload(env, codes, scales, zeros)
    Y = q4.q4_gemm_smalln_affine(c, s, z, Xd)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"affine gemm {what} M={M} K={K} N={N}")
    if N == 1:
        y = q4.q4_gemv_affine(c, s, z, Xd[0].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(Y[0], y)
    ncodes, nscales, ts, st = oracle.pack_nvfp4(W)
    assert st == 0
    Y_ref, S = oracle.gemm_nvfp4(ncodes, nscales, ts, M, K, X)
    c, s, t = _nvfp4_upload(env, ncodes, nscales, ts)
    Y = q4.q4_gemm_smalln_nvfp4(c, s, t, Xd)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"nvfp4 gemm {what} M={M} K={K} N={N}")
    if N == 1:
        y = q4.q4_gemv_nvfp4(c, s, t, Xd[0].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(Y[0], y)


@pytest.mark.parametrize("M,K,N", FMT_GEMM_CASES)
def test_gemm_smalln_formats_parity(env, M, K, N):
    seed = 9500 + M + K + N
    W = wl.weights(M, K, seed, std=0.5) + np.float32(0.03)
    if M > 3:
        W[3, :64] *= 1e-4   # subnormal NVFP4 block scales in the product
    X = wl.activations(N, K, seed, "unit_rms")
    _gemm_formats_case(env, M, K, N, W, X, "")


def _gemm_formats_ws_case(env, M, K, N, W, X, what):
    """The two formats' *_ws products against the oracle, and the same bits
    on a second call into a workspace full of NaN."""
    torch, q4, dev = env
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    ws = q4.gemm_workspace(M, K, N, dev)

    def nan_fill():
        if ws is not None:
            ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
    codes, scales, zeros, st = oracle.pack_affine(W)
    assert st == 0
    Y_ref, S = oracle.gemm_affine(codes, scales, zeros, M, K, X)
    c, s, z = _affine_upload(env, codes, scales, zeros)
    Y = q4.q4_gemm_smalln_affine_ws(c, s, z, Xd, ws).clone()
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"affine gemm ws {what} M={M} K={K} N={N}")
    nan_fill()
    assert torch.equal(Y, q4.q4_gemm_smalln_affine_ws(c, s, z, Xd, ws)), "affine: second call differs"
    ncodes, nscales, ts, st = oracle.pack_nvfp4(W)
    assert st == 0
    Y_ref, S = oracle.gemm_nvfp4(ncodes, nscales, ts, M, K, X)
    c, s, t = _nvfp4_upload(env, ncodes, nscales, ts)
    Y = q4.q4_gemm_smalln_nvfp4_ws(c, s, t, Xd, ws).clone()
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"nvfp4 gemm ws {what} M={M} K={K} N={N}")
    nan_fill()
    assert torch.equal(Y, q4.q4_gemm_smalln_nvfp4_ws(c, s, t, Xd, ws)), "nvfp4: second call differs"


@pytest.mark.parametrize("M,K,N", [(2048, 11008, 2), (70, 11008, 32), (77, 4160, 17), (301, 8256, 5),
                                   (3, 24576, 8), (300, 2048, 8)])
def test_gemm_formats_ws_parity(env, M, K, N):
    seed = 9700 + M + K + N
    W = wl.weights(M, K, seed, std=0.5) + np.float32(0.03)
    X = wl.activations(N, K, seed, "unit_rms")
    _gemm_formats_ws_case(env, M, K, N, W, X, "")


@pytest.mark.parametrize("M,K,N", [(2048, 11008, 2), (2049, 11008, 3), (77, 24576, 4), (1001, 4160, 3),
                                   (300, 8192, 4), (5, 2112, 2)])
def test_gemm_formats_tokens_long_rows_are_the_gemv(env, M, K, N):
    """Two to four tokens on rows of several waves in the affine and
    NVFP4-style formats: every token's row equals the format's GEMV of that
    token bit for bit, and the oracle within the bound (unit-RMS
    activations, as in the NF4 test above)."""
    torch, q4, dev = env
    seed = 9900 + M + K + N
    W = wl.weights(M, K, seed, std=0.5) + np.float32(0.03)
    X = wl.activations(N, K, seed, "unit_rms")
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    codes, scales, zeros, st = oracle.pack_affine(W)
    assert st == 0
    Y_ref, S = oracle.gemm_affine(codes, scales, zeros, M, K, X)
    c, s, z = _affine_upload(env, codes, scales, zeros)
    Y = q4.q4_gemm_smalln_affine(c, s, z, Xd)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"affine tokens M={M} K={K} N={N}")
    for n in range(N):
        assert torch.equal(Y[n], q4.q4_gemv_affine(c, s, z, Xd[n].contiguous())), f"affine token {n}"
    ncodes, nscales, ts, st = oracle.pack_nvfp4(W)
    assert st == 0
    Y_ref, S = oracle.gemm_nvfp4(ncodes, nscales, ts, M, K, X)
    c, s, t = _nvfp4_upload(env, ncodes, nscales, ts)
    Y = q4.q4_gemm_smalln_nvfp4(c, s, t, Xd)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"nvfp4 tokens M={M} K={K} N={N}")
    for n in range(N):
        assert torch.equal(Y[n], q4.q4_gemv_nvfp4(c, s, t, Xd[n].contiguous())), f"nvfp4 token {n}"


@pytest.mark.parametrize("M,K,N", [(77, 11008, 9), (20, 8256, 32), (300, 11008, 3), (50, 8192, 4),
                                   (2048, 11008, 2), (77, 24576, 4)])
def test_gemm_formats_ws_wide_range_activations(env, M, K, N):
    seed = 9800 + M + K + N
    W = _wide_w(wl.weights(M, K, seed, std=0.5))
    X = np.stack([_wide_x(WIDE_KINDS[(n + seed) % len(WIDE_KINDS)], K, seed + n) for n in range(N)])
    _gemm_formats_ws_case(env, M, K, N, W, X, "wide")


@pytest.mark.parametrize("M,K,N", [(300, 2048, 2), (300, 2048, 17), (77, 4160, 32), (300, 2048, 8),
                                   (3001, 1920, 5)])
def test_gemm_smalln_formats_wide_range_activations(env, M, K, N):
    seed = 9600 + M + K + N
    W = _wide_w(wl.weights(M, K, seed, std=0.5))
    X = np.stack([_wide_x(WIDE_KINDS[(n + seed) % len(WIDE_KINDS)], K, seed + n) for n in range(N)])
    _gemm_formats_case(env, M, K, N, W, X, "wide")


@pytest.mark.parametrize("shift", [0, 1])
@pytest.mark.parametrize("M,K,N", [(1001, 2048, 2), (257, 1024, 7)])
def test_gemm_smalln_affine_zero_plane_alignment(env, M, K, N, shift):
    """The affine prefill product with the zero-point plane dword-aligned
    (4-row tiles) and at 2 mod 4 (the chunk then takes the matrix-core
    kernel)."""
    torch, q4, dev = env
    seed = 3700 + M + K + N
    W = wl.weights(M, K, seed, std=0.5) + np.float32(0.03)
    X = wl.activations(N, K, seed, "unit_rms")
    codes, scales, zeros, st = oracle.pack_affine(W)
    assert st == 0
    Y_ref, S = oracle.gemm_affine(codes, scales, zeros, M, K, X)
    c, s, _ = _affine_upload(env, codes, scales, zeros)
    z = _scales_at(env, zeros, shift)
    assert z.data_ptr() % 4 == 2 * shift
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    Y = q4.q4_gemm_smalln_affine(c, s, z, Xd)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"affine gemm M={M} K={K} N={N} zero plane +{2 * shift} B")


def test_gemv_bit_exact_invariants(env):
    torch, q4, dev = env
    M, K = 1030, 2048
    W = wl.weights(M, K, 12)
    x = wl.activation(K, 12, "unit_rms")
    codes, scales, _ = oracle.pack(W)
    assert np.all(x & 0x7F80) and np.all(scales & 0x7C00)  # normal x and scales only
    c, s = _upload_packed(env, codes, scales)
    y = q4.q4_gemv(c, s, _x_dev(env, x)).cpu().numpy()
    # x * 4 (bf16 exponent + 2): y * 4 exactly
    x4 = (x.astype(np.uint32) + (2 << 7)).astype(np.uint16)
    y4 = q4.q4_gemv(c, s, _x_dev(env, x4)).cpu().numpy()
    assert np.array_equal(y4, 4 * y)
    # scales * 2 (fp16 exponent + 1): y * 2 exactly
    s2 = cases.to_dev((scales.astype(np.uint32) + (1 << 10)).astype(np.uint16).view(np.float16), torch, dev)
    y2 = q4.q4_gemv(c, s2, _x_dev(env, x)).cpu().numpy()
    assert np.array_equal(y2, 2 * y)
    # a permutation of the rows permutes y (to the acceptance bound: a row's
    # fp32 summation order depends on its slot in a row tile)
    perm = np.random.default_rng(0).permutation(M)
    cp, sp = _upload_packed(env, codes[perm], scales[perm])
    yp = q4.q4_gemv(cp, sp, _x_dev(env, x)).cpu().numpy()
    _, S = oracle.gemv(codes, scales, M, K, x)
    assert np.all(np.abs(yp - y[perm]) <= 2e-3 * S[perm] + 2e-5)
    # repeated calls are deterministic
    assert np.array_equal(q4.q4_gemv(c, s, _x_dev(env, x)).cpu().numpy(), y)


def test_gemv_no_allocation_growth(env):
    torch, q4, dev = env
    M, K = 4096, 2048
    W = wl.weights(M, K, 13)
    x = wl.activation(K, 13, "normal")
    codes, scales, _ = oracle.pack(W)
    c, s = _upload_packed(env, codes, scales)
    xd = _x_dev(env, x)
    y = torch.empty(M, dtype=torch.float32, device=dev)
    q4.q4_gemv(c, s, xd, y)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for _ in range(32):
        q4.q4_gemv(c, s, xd, y)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before


def test_gemv_on_side_stream(env):
    torch, q4, dev = env
    M, K = 512, 4096
    W = wl.weights(M, K, 14)
    x = wl.activation(K, 14, "normal")
    codes, scales, _ = oracle.pack(W)
    y_ref, S = oracle.gemv(codes, scales, M, K, x)
    c, s = _upload_packed(env, codes, scales)
    xd = _x_dev(env, x)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        y = torch.empty(M, dtype=torch.float32, device=dev)
        q4.q4_gemv(c, s, xd, y, stream=st)
    st.synchronize()
    _check(y.cpu().numpy(), y_ref, S, "gemv side stream")


def test_gemv_misaligned_device_pointer_refused(env):
    torch, q4, dev = env
    M, K = 8, 128
    codes = torch.zeros(M * K // 2 + 16, dtype=torch.uint8, device=dev)
    scales = torch.zeros((M, K // 64), dtype=torch.float16, device=dev)
    x = torch.zeros(K, dtype=torch.bfloat16, device=dev)
    bad = codes[8:8 + M * K // 2].view(M, K // 2)  # 8-byte offset
    with pytest.raises(q4.Q4Error) as e:
        q4.q4_gemv(bad, scales, x)
    assert e.value.status == q4.Q4_ERR_ALIGN


# ---------------------------------------------------------------------------
# Full-size workloads (the shapes the benchmark times), sampled rows + argmax
# ---------------------------------------------------------------------------

_FULL = {}


def _full_inputs(name):
    if name not in _FULL:
        c = wl.CONFIGS[name]
        t = time.time()
        W = wl.weights(c["M"], c["K"], c["seed"])
        _log(f"{name}: generated W {c['M']}x{c['K']} in {time.time() - t:.1f}s")
        t = time.time()
        codes, scales, st = oracle.pack(W, threads=min(16, os.cpu_count() or 1))
        _log(f"{name}: oracle pack in {time.time() - t:.1f}s")
        assert st == 0
        _FULL.clear()  # keep one full-size workload in memory at a time
        _FULL[name] = (W, codes, scales)
    return _FULL[name]


@pytest.mark.parametrize("name", ["down", "gateup", "lm_head"])
def test_full_size_pack_and_gemv(env, name):
    torch, q4, dev = env
    c = wl.CONFIGS[name]
    M, K = c["M"], c["K"]
    W, c_ref, s_ref = _full_inputs(name)
    x = wl.activation(K, c["seed"], c["x"])
    t = time.time()
    codes, scales, st = _gpu_pack(env, W)
    assert st == 0
    assert np.array_equal(codes.cpu().numpy(), c_ref), "pack codes differ"
    assert np.array_equal(cases.bits16(scales, torch), s_ref), "pack scales differ"
    _log(f"{name}: GPU pack bit-exact ({time.time() - t:.1f}s incl. upload)")
    y = q4.q4_gemv(codes, scales, _x_dev(env, x)).cpu().numpy()
    t = time.time()
    y_full, S_full = oracle.gemv(c_ref, s_ref, M, K, x, threads=min(16, os.cpu_count() or 1))
    _log(f"{name}: full oracle GEMV in {time.time() - t:.1f}s")
    _check(y, y_full, S_full, f"{name} all {M} rows")
    if name == "lm_head":
        a_ref = oracle.argmax(y_full)
        a_gpu = oracle.argmax(y)
        top = np.sort(y_full)[-2:]
        _log(f"lm_head argmax gpu={a_gpu} oracle={a_ref} top-2 gap={top[1] - top[0]:.4g}")
        assert a_gpu == a_ref


# ---------------------------------------------------------------------------
# q4_gemm_smalln
# ---------------------------------------------------------------------------

# (M, K, N): ragged row tiles (16 rows), K slices of 256 (partial last
# slices; up to 8 slices the activations stay in registers, beyond that each
# wave reloads its slices per tile), one or two 16-token halves, and enough
# tiles per workgroup (20000 rows) that the prefetch ring wraps; 40000 rows
# give each workgroup several groups of tiles between the cross-wave sums.
GEMM_SHAPES = [(1, 64, 1), (40, 128, 2), (100, 512, 3), (64, 2048, 4), (97, 1024, 8),
               (33, 2048, 16), (200, 2048, 17), (65, 4096, 31), (160, 2048, 32), (70, 11008, 32),
               (300, 1600, 20), (50, 2112, 32), (20000, 256, 9), (20000, 192, 32),
               (40000, 64, 5), (40000, 128, 24),
               # one token takes the GEMV kernels (short and long rows)
               (7, 2048, 1), (3000, 2112, 1), (600, 11008, 1),
               # two to eight tokens on short rows take 4-row tiles (up to
               # 12 a CU; K % 128 == 0), two or three with K % 128 == 64 the
               # GEMV with shared lookups, beyond that the matrix-core kernel
               (11008, 2048, 2), (3001, 1984, 3), (5, 64, 2), (1001, 576, 3), (12289, 2048, 3),
               # every matrix-core instantiation: two tokens past the
               # shared-lookup GEMV's limit (activations in registers, one
               # token pair loaded), and long rows with 1, 2, 4, 8 token pairs
               # in one half and 12 in two halves
               (12293, 2048, 2), (70, 11008, 2), (65, 4096, 3), (97, 4160, 8), (33, 11008, 16),
               (50, 2112, 20),
               # odd blocks a row with a last tile reaching past M, and 15
               # tiles a workgroup
               (3000, 1984, 32), (3000, 1984, 4), (3001, 1984, 17), (3001, 1984, 4), (60000, 2048, 8),
               # 2..4 tokens on 4-row tiles: rows not a multiple of 4, K not
               # a multiple of 512 (a partial activation range), one row,
               # the most tiles a launch takes (12 a CU), the fewest waves
               (3001, 1920, 4), (12288, 2048, 4), (1, 128, 2), (13, 640, 3), (4099, 1152, 2),
               (3001, 1920, 2),
               # 5..8 tokens on 4-row tiles (two token groups), and 9..16
               # tokens on the same shapes (the 16-row matrix-core kernel)
               (3001, 1920, 8), (12288, 2048, 7), (13, 640, 7), (4099, 1152, 6), (2, 256, 5),
               (3001, 1920, 16), (12288, 2048, 13), (2, 256, 16),
               # two to four tokens on rows of several waves: the grouped
               # GEMV with shared lookups (2 and 3 tokens on rows of 65..768
               # chunks, 4 tokens from 256 chunks), both sides of each limit,
               # ragged row counts, scale planes without one-load scale runs
               (64, 8128, 4), (64, 8192, 4), (40, 24576, 3), (40, 24640, 3), (3, 2112, 3),
               (4099, 4160, 2), (2049, 11008, 3), (1, 11008, 4), (9001, 4096, 2)]


@pytest.mark.parametrize("M,K,N", GEMM_SHAPES)
def test_gemm_smalln_parity(env, M, K, N):
    torch, q4, dev = env
    seed = 3000 + M + K + N
    W = wl.weights(M, K, seed)
    X = wl.activations(N, K, seed, "unit_rms")
    codes, scales, _ = oracle.pack(W)
    Y_ref, S = oracle.gemm(codes, scales, M, K, X)
    c, s = _upload_packed(env, codes, scales)
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    Y = q4.q4_gemm_smalln(c, s, Xd)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"gemm M={M} K={K} N={N}")


@pytest.mark.parametrize("shift", [0, 1])
@pytest.mark.parametrize("M,K,N", [(1001, 2048, 2), (300, 1024, 3), (4099, 1152, 4), (257, 2048, 8)])
def test_gemm_smalln_scale_plane_alignment(env, M, K, N, shift):
    """2..8 tokens with the scale plane dword-aligned (4-row tiles) and at
    2 mod 4 (the 4-row-tile kernel needs dword-aligned scales: the chunk
    then takes the shared-lookup GEMV or the matrix-core kernel)."""
    torch, q4, dev = env
    seed = 3500 + M + K + N
    W = wl.weights(M, K, seed)
    X = wl.activations(N, K, seed, "unit_rms")
    codes, scales, _ = oracle.pack(W)
    Y_ref, S = oracle.gemm(codes, scales, M, K, X)
    c, _ = _upload_packed(env, codes, scales)
    s = _scales_at(env, scales, shift)
    assert s.data_ptr() % 4 == 2 * shift
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    Y = q4.q4_gemm_smalln(c, s, Xd)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"gemm M={M} K={K} N={N} scale plane +{2 * shift} B")


def test_gemm_one_token_is_the_gemv(env):
    """A one-token chunk runs the GEMV kernels: bit-identical to q4_gemv."""
    torch, q4, dev = env
    for M, K in ((300, 2048), (257, 11008)):
        W = wl.weights(M, K, 43)
        X = wl.activations(1, K, 43, "unit_rms")
        codes, scales, _ = oracle.pack(W)
        c, s = _upload_packed(env, codes, scales)
        Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
        Y = q4.q4_gemm_smalln(c, s, Xd)
        y = q4.q4_gemv(c, s, Xd[0].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(Y[0], y), f"M={M} K={K}"


def test_gemm_rows_match_gemv(env):
    torch, q4, dev = env
    M, K, N = 300, 2048, 5
    W = wl.weights(M, K, 41)
    X = wl.activations(N, K, 41, "normal")
    codes, scales, _ = oracle.pack(W)
    c, s = _upload_packed(env, codes, scales)
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    Y = q4.q4_gemm_smalln(c, s, Xd).cpu().numpy()
    for n in range(N):
        y = q4.q4_gemv(c, s, Xd[n].contiguous()).cpu().numpy()
        _, Sn = oracle.gemv(codes, scales, M, K, X[n])
        assert np.all(np.abs(Y[n] - y) <= 2e-3 * Sn + 2e-5)


def test_gemm_smalln_full_size(env):
    """The prefill shape (11008 x 2048), chunks of 32 .. 1 tokens, every
    output against the oracle."""
    torch, q4, dev = env
    c = wl.CONFIGS["smalln"]
    M, K, N = c["M"], c["K"], c["N"]
    W = wl.weights(M, K, c["seed"])
    X = wl.activations(N, K, c["seed"], c["x"])
    codes, scales, st = _gpu_pack(env, W)
    assert st == 0
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    c_ref, s_ref, _ = oracle.pack(W, threads=min(16, os.cpu_count() or 1))
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    t = time.time()
    Y_ref, S = oracle.gemm(c_ref, s_ref, M, K, X)
    _log(f"smalln: oracle product of {N} tokens in {time.time() - t:.1f}s")
    for n_tok in (32, 17, 16, 8, 4, 3, 2, 1):
        Y = q4.q4_gemm_smalln(codes, scales, Xd[:n_tok].contiguous()).cpu().numpy()
        _check(Y, Y_ref[:n_tok], S[:n_tok], f"smalln N={n_tok} all {M} rows")


@pytest.mark.parametrize("M,K,N", [(2048, 11008, 2), (2049, 11008, 3), (1001, 4160, 3), (77, 24576, 4),
                                   (300, 8192, 4), (20000, 4096, 2), (5, 2112, 2)])
def test_gemm_tokens_long_rows_are_the_gemv(env, M, K, N):
    """Two to four tokens on rows of several waves: every token's row equals
    q4_gemv of that token bit for bit (the same conversion, products,
    reduction and cross-wave sum per token), and the oracle within the bound.
    (Unit-RMS activations: no wave's values span more than 2^28, so every
    wave takes the fp16 path for every token, as the GEMV does; a wave with
    one token beyond that takes the exact path for all of them.)"""
    torch, q4, dev = env
    seed = 8200 + M + K + N
    W = wl.weights(M, K, seed)
    X = wl.activations(N, K, seed, "unit_rms")
    codes, scales, _ = oracle.pack(W)
    Y_ref, S = oracle.gemm(codes, scales, M, K, X)
    c, s = _upload_packed(env, codes, scales)
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    Y = q4.q4_gemm_smalln(c, s, Xd)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"gemm tokens M={M} K={K} N={N}")
    for n in range(N):
        y = q4.q4_gemv(c, s, Xd[n].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(Y[n], y), f"token {n} of M={M} K={K} N={N} differs from its GEMV"


def test_gemm_smalln_full_size_down(env):
    """The prefill product on the down projection's shape (2048 x 11008):
    chunks of 32, 8, 4, 3 and 2 tokens (the 16-row kernel on long rows, and
    the grouped GEMV with shared lookups), every output against the oracle."""
    torch, q4, dev = env
    c = wl.CONFIGS["down"]
    M, K, N = c["M"], c["K"], 32
    W = wl.weights(M, K, c["seed"])
    X = wl.activations(N, K, c["seed"], c["x"])
    codes, scales, st = _gpu_pack(env, W)
    assert st == 0
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    c_ref, s_ref, _ = oracle.pack(W, threads=min(16, os.cpu_count() or 1))
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    t = time.time()
    Y_ref, S = oracle.gemm(c_ref, s_ref, M, K, X)
    _log(f"down prefill: oracle product of {N} tokens in {time.time() - t:.1f}s")
    for n_tok in (32, 8, 4, 3, 2):
        Y = q4.q4_gemm_smalln(codes, scales, Xd[:n_tok].contiguous()).cpu().numpy()
        _check(Y, Y_ref[:n_tok], S[:n_tok], f"down prefill N={n_tok} all {M} rows")
    # With scratch memory: K split in six ranges (chunks of 5..32 tokens).
    for n_tok in (32, 16, 8, 5):
        ws = q4.gemm_workspace(M, K, n_tok, dev)
        assert ws is not None
        Y = q4.q4_gemm_smalln_ws(codes, scales, Xd[:n_tok].contiguous(), ws).cpu().numpy()
        _check(Y, Y_ref[:n_tok], S[:n_tok], f"down prefill with scratch N={n_tok} all {M} rows")


WS_SHAPES = [(2048, 11008, 5), (70, 11008, 32), (4099, 4160, 9), (33, 11008, 16), (1, 2112, 5),
             (3, 131072, 32), (77, 24576, 17), (5120, 5120, 4), (301, 8256, 12), (2, 4160, 2)]


@pytest.mark.parametrize("M,K,N", WS_SHAPES)
def test_gemm_ws_parity(env, M, K, N):
    """q4_gemm_smalln_ws: K split in ranges of at most 2048 weights on long
    rows (or q4_gemm_smalln where no scratch is needed), every output against
    the oracle; the same bits on a second call into a workspace full of NaN."""
    torch, q4, dev = env
    seed = 8800 + M + K + N
    W = wl.weights(M, K, seed)
    X = wl.activations(N, K, seed, "unit_rms")
    codes, scales, _ = oracle.pack(W)
    Y_ref, S = oracle.gemm(codes, scales, M, K, X)
    c, s = _upload_packed(env, codes, scales)
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    ws = q4.gemm_workspace(M, K, N, dev)
    Y = q4.q4_gemm_smalln_ws(c, s, Xd, ws).clone()
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"gemm ws M={M} K={K} N={N}")
    if ws is not None:
        ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
    Y2 = q4.q4_gemm_smalln_ws(c, s, Xd, ws)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2), f"M={M} K={K} N={N}: second call differs"
    if ws is None:
        assert torch.equal(Y, q4.q4_gemm_smalln(c, s, Xd)), "no scratch: the call is q4_gemm_smalln"


@pytest.mark.parametrize("M,K,N", [(300, 11008, 8), (77, 4160, 17), (20, 24576, 32)])
def test_gemm_ws_wide_range_activations(env, M, K, N):
    """The split's ranges each take their own exact or fp16 path per wave."""
    torch, q4, dev = env
    seed = 8900 + M + K + N
    W = _wide_w(wl.weights(M, K, seed))
    X = np.stack([_wide_x(WIDE_KINDS[(n + seed) % len(WIDE_KINDS)], K, seed + n) for n in range(N)])
    codes, scales, _ = oracle.pack(W)
    Y_ref, S = oracle.gemm(codes, scales, M, K, X)
    c, s = _upload_packed(env, codes, scales)
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    Y = q4.q4_gemm_smalln_ws(c, s, Xd, q4.gemm_workspace(M, K, N, dev))
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, S, f"gemm ws wide M={M} K={K} N={N}")


def test_gemm_formats_full_size_down(env):
    """The affine and NVFP4-style prefill products on the down projection's
    shape (2048 x 11008): 2 and 4 tokens (the grouped GEMV with shared
    lookups) and 8 and 32 tokens with scratch (the K split), every output
    against the oracle."""
    torch, q4, dev = env
    c = wl.CONFIGS["down"]
    M, K, N = c["M"], c["K"], 32
    W = wl.weights(M, K, c["seed"])
    X = wl.activations(N, K, c["seed"], c["x"])
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    codes, scales, zeros, st = oracle.pack_affine(W)
    assert st == 0
    Y_ref, S = oracle.gemm_affine(codes, scales, zeros, M, K, X)
    ca, sa, za = _affine_upload(env, codes, scales, zeros)
    ncodes, nscales, ts, st = oracle.pack_nvfp4(W)
    assert st == 0
    Yn_ref, Sn = oracle.gemm_nvfp4(ncodes, nscales, ts, M, K, X)
    cn, sn, tn = _nvfp4_upload(env, ncodes, nscales, ts)
    ws = q4.gemm_workspace(M, K, N, dev)
    for n_tok in (32, 8, 4, 2):
        Xn = Xd[:n_tok].contiguous()
        Y = q4.q4_gemm_smalln_affine_ws(ca, sa, za, Xn, ws).cpu().numpy()
        _check(Y, Y_ref[:n_tok], S[:n_tok], f"affine down prefill N={n_tok} all {M} rows")
        Y = q4.q4_gemm_smalln_nvfp4_ws(cn, sn, tn, Xn, ws).cpu().numpy()
        _check(Y, Yn_ref[:n_tok], Sn[:n_tok], f"nvfp4 down prefill N={n_tok} all {M} rows")


def test_graph_capture_long_row_tokens(env):
    """The grouped GEMV with shared lookups (2, 3 and 4 tokens on rows of
    11008 weights) and the K split with scratch (9 tokens) captured in a HIP
    graph equal eager on every replay."""
    torch, q4, dev = env
    M, K = 600, 11008
    W = wl.weights(M, K, 53)
    codes, scales, _ = oracle.pack(W)
    c, s = _upload_packed(env, codes, scales)
    Xs = [cases.to_dev(wl.activations(n, K, 53 + n, "swiglu").view(np.int16), torch, dev).view(torch.bfloat16)
          for n in (2, 3, 4)]
    X9 = cases.to_dev(wl.activations(9, K, 59, "swiglu").view(np.int16), torch, dev).view(torch.bfloat16)
    ws = q4.gemm_workspace(M, K, 9, dev)
    eager = [q4.q4_gemm_smalln(c, s, X).clone() for X in Xs] + [q4.q4_gemm_smalln_ws(c, s, X9, ws).clone()]
    outs = [torch.full((X.shape[0], M), float("nan"), device=dev) for X in Xs + [X9]]
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            for X, Y in zip(Xs, outs):
                q4.q4_gemm_smalln(c, s, X, Y, stream=st)
            # nine tokens with scratch: the K split and the sum of its planes
            q4.q4_gemm_smalln_ws(c, s, X9, ws, outs[-1], stream=st)
    torch.cuda.synchronize()
    for rep in range(4):
        for Y in outs:
            Y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for Y, E in zip(outs, eager):
            assert torch.equal(Y, E), f"long-row {Y.shape[0]}-token replay {rep} differs from eager"
        q4.q4_gemm_smalln(c, s, Xs[0])
        torch.cuda.synchronize()


def test_gemm_formats_full_size(env):
    """The prefill shape (11008 x 2048) in the affine and NVFP4-style
    formats, packed by the oracle: chunks of 32, 17, 8, 5, 4 and 2 tokens
    (the 16-row and the 4-row-tile kernels, in the launch configuration
    bench.py times), every output against the oracle."""
    torch, q4, dev = env
    c = wl.CONFIGS["smalln"]
    M, K, N = c["M"], c["K"], c["N"]
    W = wl.weights(M, K, c["seed"])
    X = wl.activations(N, K, c["seed"], c["x"])
    Xd = cases.to_dev(X.view(np.int16), torch, dev).view(torch.bfloat16)
    threads = min(16, os.cpu_count() or 1)
    codes, scales, zeros, st = oracle.pack_affine(W, threads=threads)
    assert st == 0
    Y_ref, S = oracle.gemm_affine(codes, scales, zeros, M, K, X, threads=threads)
    cd, sd, zd = _affine_upload(env, codes, scales, zeros)
    for n_tok in (32, 17, 8, 5, 4, 2):
        Y = q4.q4_gemm_smalln_affine(cd, sd, zd, Xd[:n_tok].contiguous()).cpu().numpy()
        _check(Y, Y_ref[:n_tok], S[:n_tok], f"affine smalln N={n_tok} all {M} rows")
    ncodes, nscales, ts, st = oracle.pack_nvfp4(W, threads=threads)
    assert st == 0
    Y_ref, S = oracle.gemm_nvfp4(ncodes, nscales, ts, M, K, X, threads=threads)
    cd, sd, td = _nvfp4_upload(env, ncodes, nscales, ts)
    for n_tok in (32, 17, 8, 5, 4, 2):
        Y = q4.q4_gemm_smalln_nvfp4(cd, sd, td, Xd[:n_tok].contiguous()).cpu().numpy()
        _check(Y, Y_ref[:n_tok], S[:n_tok], f"nvfp4 smalln N={n_tok} all {M} rows")


# ---------------------------------------------------------------------------
# HIP graph capture (a decode step is captured once and replayed)
# ---------------------------------------------------------------------------

def test_graph_capture_strided_and_grouped_launches(env):
    """The strided short-row launch (more than 16 tiles per CU) and the
    grouped long-row launch, captured in one graph: every replay equals the
    eager result bit for bit."""
    torch, q4, dev = env
    outs, calls = [], []
    for M, K in ((40000, 2048), (3000, 5120)):
        W = wl.weights(M, K, 52)
        codes, scales, _ = oracle.pack(W)
        c, s = _upload_packed(env, codes, scales)
        x = _x_dev(env, wl.activation(K, 52, "unit_rms"))
        y_eager = q4.q4_gemv(c, s, x).clone()
        y = torch.full((M,), float("nan"), device=dev)
        outs.append((y, y_eager))
        calls.append((c, s, x, y))
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            for c, s, x, y in calls:
                q4.q4_gemv(c, s, x, y, stream=st)
    torch.cuda.synchronize()
    for rep in range(3):
        for y, _ in outs:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, y_eager) in enumerate(outs):
            assert torch.equal(y, y_eager), f"launch {i} replay {rep} differs from eager"


def test_graph_capture_replays_match_eager(env):
    torch, q4, dev = env
    M, K, N = 3000, 2048, 16
    W = wl.weights(M, K, 51)
    codes, scales, _ = oracle.pack(W)
    c, s = _upload_packed(env, codes, scales)
    x = _x_dev(env, wl.activation(K, 51, "unit_rms"))
    X = cases.to_dev(wl.activations(N, K, 51, "normal").view(np.int16), torch, dev).view(torch.bfloat16)
    X2 = X[:2].contiguous()  # two tokens: 4-row tiles, one token group
    X8 = X[:8].contiguous()  # eight tokens: 4-row tiles, two token groups
    # (sixteen tokens: the 16-row matrix-core kernel)
    y_eager = q4.q4_gemv(c, s, x).clone()
    Y_eager = q4.q4_gemm_smalln(c, s, X).clone()
    Y2_eager = q4.q4_gemm_smalln(c, s, X2).clone()
    Y8_eager = q4.q4_gemm_smalln(c, s, X8).clone()
    y = torch.full((M,), float("nan"), device=dev)
    Y = torch.full((N, M), float("nan"), device=dev)
    Y2 = torch.full((2, M), float("nan"), device=dev)
    Y8 = torch.full((8, M), float("nan"), device=dev)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            q4.q4_gemv(c, s, x, y, stream=st)
            q4.q4_gemm_smalln(c, s, X, Y, stream=st)
            q4.q4_gemm_smalln(c, s, X2, Y2, stream=st)
            q4.q4_gemm_smalln(c, s, X8, Y8, stream=st)
    torch.cuda.synchronize()
    for rep in range(4):
        y.fill_(float("nan"))
        Y.fill_(float("nan"))
        Y2.fill_(float("nan"))
        Y8.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"gemv replay {rep} differs from eager"
        assert torch.equal(Y, Y_eager), f"gemm replay {rep} differs from eager"
        assert torch.equal(Y2, Y2_eager), f"two-token gemm replay {rep} differs from eager"
        assert torch.equal(Y8, Y8_eager), f"eight-token gemm replay {rep} differs from eager"
        # eager work in between replays
        q4.q4_gemv(c, s, x)
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# q4_gemv_fused: several products of one x with the decode epilogues
# ---------------------------------------------------------------------------

EPS32 = 2.0 ** -24


def _fused_ref(ts, Ss, biases, residuals, swiglu):
    """Oracle outputs and per-element bounds for the fused epilogue.

    Each product t_i carries the GEMV bound e_i = 1e-3 S_i + 1e-5; the fp32
    adds of bias and residual each add at most one rounding (half an ulp,
    counted here as a full EPS32 of the operands).  SwiGLU: silu has slope in
    (-0.1, 1.1), so an error e_a in its argument moves silu by at most 1.1 e_a;
    the product silu(a) * b then moves by 1.1 e_a (|b| + e_b) + |silu(a)| e_b,
    and the fp32 exp, divide and multiplies add a few ulps of |silu(a) b|."""
    f64 = lambda v: None if v is None else np.asarray(v, np.float64)
    if swiglu:
        y = oracle.epilogue(ts[0], ts[1], biases[0], biases[1], residuals[0], swiglu=True)
        b0, b1 = f64(biases[0]), f64(biases[1])
        a = ts[0] + (b0 if b0 is not None else 0.0)
        b = ts[1] + (b1 if b1 is not None else 0.0)
        ea = 1e-3 * Ss[0] + 1e-5 + EPS32 * np.abs(a)
        eb = 1e-3 * Ss[1] + 1e-5 + EPS32 * np.abs(b)
        sa = np.array([oracle.silu(v) for v in a]) if a.size <= 4096 else a / (1.0 + np.exp(-a))
        r = f64(residuals[0])
        bound = 1.1 * ea * (np.abs(b) + eb) + np.abs(sa) * eb + 8 * EPS32 * (
            np.abs(sa * b) + (np.abs(r) if r is not None else 0.0))
        return [y], [bound]
    ys, bounds = [], []
    for t, S, bias, res in zip(ts, Ss, biases, residuals):
        ys.append(oracle.epilogue(t, bias0=bias, residual=res))
        mag = np.abs(t) + (np.abs(f64(bias)) if bias is not None else 0.0) + (
            np.abs(f64(res)) if res is not None else 0.0)
        bounds.append(1e-3 * S + 1e-5 + 2 * EPS32 * mag)
    return ys, bounds


def _check_bound(y_gpu, y_ref, bound, what):
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ref)
    ratio = float(np.max(err / bound)) if err.size else 0.0
    _log(f"{what}: worst |err|/bound = {ratio:.3g}")
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    assert np.all(err <= bound), f"{what}: tolerance broken, worst ratio {ratio}"


def _fused_case(env, Ms, K, seed, swiglu=False, bias=True, residual=True, alias=(), x_recipe="unit_rms",
                bias_scale=0.5, x=None, w_hook=None, fmt="nf4"):
    """Packs len(Ms) matrices in format `fmt` ("nf4", "affine", "nvfp4"),
    runs the format's fused entry point, checks every output against the
    oracle and against the format's unfused GEMV followed by torch's
    epilogue.  `x` (bf16 bits) replaces the recipe's activations; `w_hook(W)`
    edits each fp32 matrix before it is packed."""
    torch, q4, dev = env
    if x is None:
        x = wl.activation(K, seed, x_recipe)
    xd = _x_dev(env, x)
    ops, ts, Ss, biases, packed = [], [], [], [], []
    rng = np.random.default_rng(seed)
    for i, M in enumerate(Ms):
        W = wl.weights(M, K, seed + 17 * i)
        if w_hook is not None:
            W = w_hook(W)
        if fmt == "affine":
            codes, scales, zeros, st = oracle.pack_affine(W)
            t, S = oracle.gemv_affine(codes, scales, zeros, M, K, x)
            dev_ops = _affine_upload(env, codes, scales, zeros)
        elif fmt == "nvfp4":
            codes, scales, tsv, st = oracle.pack_nvfp4(W)
            t, S = oracle.gemv_nvfp4(codes, scales, tsv, M, K, x)
            dev_ops = _nvfp4_upload(env, codes, scales, tsv)
        else:
            codes, scales, st = oracle.pack(W)
            t, S = oracle.gemv(codes, scales, M, K, x)
            dev_ops = _upload_packed(env, codes, scales)
        assert st == 0
        b = (rng.standard_normal(M) * bias_scale).astype(np.float32) if bias else None
        bd = torch.from_numpy(b).to(dev) if b is not None else None
        ops.append(tuple(dev_ops) + (bd,))
        ts.append(t)
        Ss.append(S)
        biases.append(b)
        packed.append(tuple(dev_ops))
    nout = 1 if swiglu else len(Ms)
    res_h = [(rng.standard_normal(Ms[o]) * 2).astype(np.float32) if residual else None for o in range(nout)]
    ys = [torch.full((Ms[o],), float("nan"), device=dev) for o in range(nout)]
    res_d = []
    for o in range(nout):
        if res_h[o] is None:
            res_d.append(None)
        elif o in alias:  # in-place: the output buffer holds the residual
            ys[o].copy_(torch.from_numpy(res_h[o]))
            res_d.append(ys[o])
        else:
            res_d.append(torch.from_numpy(res_h[o]).to(dev))
    fused = {"nf4": q4.q4_gemv_fused, "affine": q4.q4_gemv_fused_affine, "nvfp4": q4.q4_gemv_fused_nvfp4}[fmt]
    gemv = {"nf4": q4.q4_gemv, "affine": q4.q4_gemv_affine, "nvfp4": q4.q4_gemv_nvfp4}[fmt]
    fused(ops, xd, "swiglu" if swiglu else "separate", ys, res_d if residual else None)
    torch.cuda.synchronize()
    y_ref, bound = _fused_ref(ts, Ss, biases, res_h, swiglu)
    what = f"{fmt} fused {'swiglu' if swiglu else 'separate'} Ms={Ms} K={K}"
    for o in range(nout):
        _check_bound(ys[o].cpu().numpy(), y_ref[o], bound[o], f"{what} out {o}")
    # Unfused: one q4_gemv per matrix, then torch's epilogue in fp32.
    tg = [gemv(*p, xd) for p in packed]
    for i in range(len(tg)):
        if biases[i] is not None:
            tg[i] = tg[i] + ops[i][-1]
    if swiglu:
        un = [torch.nn.functional.silu(tg[0]) * tg[1]]
    else:
        un = tg
    for o in range(nout):
        if res_h[o] is not None:
            un[o] = un[o] + torch.from_numpy(res_h[o]).to(dev)
        torch.cuda.synchronize()
        # both sides are within `bound` of the oracle
        _check_bound(ys[o].cpu().numpy(), un[o].cpu().numpy().astype(np.float64), 2 * bound[o],
                     f"{what} out {o} vs unfused")
    return ys


# (Ms, K): the row-length classes of the launcher (one wave a row up to
# K=2048, two chunks a lane to 4096, a workgroup a row to 16384), segments of
# ragged and empty sizes, and single-tile and ring plans.
FUSED_SEPARATE = [((2048, 256, 256), 2048), ((1, 65, 0, 300), 512), ((7,), 64), ((4096, 4096), 2048),
                  ((33, 1000, 2), 4096), ((2048,), 11008), ((129, 5, 4100), 4160), ((40, 3), 16384),
                  ((20000, 300), 1024)]


@pytest.mark.parametrize("Ms,K", FUSED_SEPARATE)
def test_fused_separate_bias_residual(env, Ms, K):
    _fused_case(env, Ms, K, seed=5000 + K + sum(Ms))


@pytest.mark.parametrize("bias,residual", [(False, False), (True, False), (False, True)])
def test_fused_separate_optional_terms(env, bias, residual):
    _fused_case(env, (300, 64, 1), 2048, seed=5100, bias=bias, residual=residual)


def test_fused_residual_in_place(env):
    # down projection with the residual stream updated in place, plus a
    # second output that is not aliased
    _fused_case(env, (2048, 77), 11008, seed=5200, alias=(0,))
    _fused_case(env, (513, 1, 64), 2048, seed=5201, alias=(0, 2))


# (M, K): gate/up pairs over the same row-length classes.
FUSED_SWIGLU = [(11008, 2048), (1, 64), (77, 512), (5000, 2048), (300, 4096), (2048, 4160),
                (129, 11008), (20, 16384), (20000, 1024)]


@pytest.mark.parametrize("M,K", FUSED_SWIGLU)
def test_fused_swiglu(env, M, K):
    _fused_case(env, (M, M), K, seed=6000 + M + K, swiglu=True)


@pytest.mark.parametrize("bias,residual,alias", [(False, False, ()), (True, False, ()), (False, True, (0,))])
def test_fused_swiglu_optional_terms(env, bias, residual, alias):
    _fused_case(env, (1100, 1100), 2048, seed=6100, swiglu=True, bias=bias, residual=residual, alias=alias)


def test_fused_swiglu_wide_activations(env):
    # gate biases of tens drive silu into both tails (e^-z overflows to inf
    # for z < -88)
    _fused_case(env, (500, 500), 2048, seed=6200, swiglu=True, x_recipe="normal", bias_scale=60.0)


# The fused forms of the affine and NVFP4-style formats: the launcher's
# row-length classes (one wave a row, a workgroup a row), ragged and empty
# segments, the strided order (11008 x 2048 SwiGLU), one-tile and ring plans,
# an in-place residual.  Each NVFP4-style matrix has its own tensor scale.
FUSED_FMT_SEPARATE = [((2048, 256, 256), 2048), ((1, 65, 0, 300), 512), ((2048,), 11008), ((33, 1000, 2), 4096),
                      ((20000, 300), 1024), ((129, 5, 4100), 4160)]
FUSED_FMT_SWIGLU = [(11008, 2048), (77, 512), (5000, 2048), (129, 11008), (300, 4096), (20000, 1024), (1, 64)]


@pytest.mark.parametrize("fmt", ["affine", "nvfp4"])
@pytest.mark.parametrize("Ms,K", FUSED_FMT_SEPARATE)
def test_fused_formats_separate(env, fmt, Ms, K):
    _fused_case(env, Ms, K, seed=5300 + K + sum(Ms), fmt=fmt, alias=(0,) if K == 11008 else ())


@pytest.mark.parametrize("fmt", ["affine", "nvfp4"])
@pytest.mark.parametrize("M,K", FUSED_FMT_SWIGLU)
def test_fused_formats_swiglu(env, fmt, M, K):
    _fused_case(env, (M, M), K, seed=6400 + M + K, swiglu=True, fmt=fmt)


@pytest.mark.parametrize("fmt", ["affine", "nvfp4"])
@pytest.mark.parametrize("kind", ["code7_column_2^60", "spread_32"])
@pytest.mark.parametrize("swiglu,Ms,K", [(False, (2048, 256, 256), 2048), (True, (1000, 1000), 2048),
                                         (True, (300, 300), 4160)])
def test_fused_formats_wide_range_activations(env, fmt, swiglu, Ms, K, kind):
    """Activations past the fp16 conversion's range: the exact loop, with
    the up matrix's own zero points and tensor scale in the SwiGLU form."""
    seed = 7700 + K + sum(Ms)
    _fused_case(env, Ms, K, seed, swiglu=swiglu, x=_wide_x(kind, K, seed), w_hook=_wide_w, bias_scale=1e-3, fmt=fmt)


@pytest.mark.parametrize("M,K", [(1101, 576), (1100, 1024), (9001, 192)])
def test_fused_affine_swiglu_planes_of_one_matrix(env, M, K):
    """Affine gate and up as the halves of one packed matrix: with an odd M
    or an odd number of blocks a row the up half's scale and zero-point
    planes sit at 2 mod 4, and the launch reads them per row."""
    torch, q4, dev = env
    W = wl.weights(2 * M, K, 6600 + M) + np.float32(0.02)
    x = wl.activation(K, 6600 + M, "unit_rms")
    codes, scales, zeros, st = oracle.pack_affine(W)
    assert st == 0
    t, S = oracle.gemv_affine(codes, scales, zeros, 2 * M, K, x)
    c, s, z = _affine_upload(env, codes, scales, zeros)
    _log(f"affine swiglu M={M} K={K}: up planes at {s[M:].data_ptr() % 4}, {z[M:].data_ptr() % 4} mod 4")
    ops = [(c[:M], s[:M], z[:M], None), (c[M:], s[M:], z[M:], None)]
    y = q4.q4_gemv_fused_affine(ops, _x_dev(env, x), "swiglu")[0]
    torch.cuda.synchronize()
    y_ref, bound = _fused_ref([t[:M], t[M:]], [S[:M], S[M:]], [None, None], [None], True)
    _check_bound(y.cpu().numpy(), y_ref[0], bound[0], f"affine swiglu halves M={M} K={K}")


def test_fused_swiglu_halves_of_one_matrix(env):
    """Gate and up packed as one [2M, K] matrix: the two operands are the
    halves of one codes/scales buffer."""
    torch, q4, dev = env
    M, K = 1100, 2048
    W = wl.weights(2 * M, K, 6300)
    x = wl.activation(K, 6300, "unit_rms")
    codes, scales, _ = oracle.pack(W)
    t, S = oracle.gemv(codes, scales, 2 * M, K, x)
    c, s = _upload_packed(env, codes, scales)
    ops = [(c[:M], s[:M], None), (c[M:], s[M:], None)]
    y = q4.q4_gemv_fused(ops, _x_dev(env, x), "swiglu")[0]
    torch.cuda.synchronize()
    y_ref, bound = _fused_ref([t[:M], t[M:]], [S[:M], S[M:]], [None, None], [None], True)
    _check_bound(y.cpu().numpy(), y_ref[0], bound[0], "swiglu halves")


def test_fused_graph_replays_match_eager(env):
    torch, q4, dev = env
    K = 2048
    ops, packed = [], []
    for i, M in enumerate((2048, 256, 256)):
        codes, scales, _ = oracle.pack(wl.weights(M, K, 6400 + i))
        c, s = _upload_packed(env, codes, scales)
        ops.append((c, s, torch.randn(M, device=dev)))
    x = _x_dev(env, wl.activation(K, 6400, "unit_rms"))
    eager = [v.clone() for v in q4.q4_gemv_fused(ops, x)]
    ys = [torch.full_like(v, float("nan")) for v in eager]
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            q4.q4_gemv_fused(ops, x, "separate", ys, stream=st)
    torch.cuda.synchronize()
    for rep in range(3):
        for v in ys:
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ys, eager):
            assert torch.equal(a, b), f"fused replay {rep} differs from eager"
        q4.q4_gemv_fused(ops, x)
        torch.cuda.synchronize()


def test_fused_rejects_through_binding(env):
    torch, q4, dev = env
    K = 128
    codes, scales, _ = oracle.pack(wl.weights(8, K, 1))
    c, s = _upload_packed(env, codes, scales)
    x = _x_dev(env, wl.activation(K, 1, "unit_rms"))
    with pytest.raises(q4.Q4Error):
        q4.q4_gemv_fused([(c, s, None)] * 3, x, "swiglu")
    y = torch.empty(8, device=dev)
    with pytest.raises(q4.Q4Error):  # residual overlapping its output off by one element
        big = torch.zeros(9, device=dev)
        q4.q4_gemv_fused([(c, s, None)], x, "separate", [big[:8]], [big[1:]])
    del y


# ---------------------------------------------------------------------------
# q4_gather_rows: packed rows dequantised (bit-exact: one rounding of the
# exact level * scale on both sides)
# ---------------------------------------------------------------------------

# (M, K, n): one and several workgroups per row (K/4 or K/8 lanes of 256),
# ragged last workgroups (K = 11008: 2752 / 1376 lanes), repeated ids.
GATHER_SHAPES = [(1, 64, 1), (37, 192, 6), (300, 2048, 32), (257, 4160, 5), (64, 11008, 9), (9, 16384, 3)]


def _gather_case(env, M, K, n, seed, dtype_name):
    torch, q4, dev = env
    bf16 = dtype_name == "bf16"
    W = wl.weights(M, K, seed, std=0.5)
    codes, scales, st = oracle.pack(W)
    assert st == 0
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, M, n).astype(np.int32)
    ref, flags = oracle.gather_rows(codes, scales, M, K, ids, bf16=bf16)
    assert flags == 0
    c, s = _upload_packed(env, codes, scales)
    idd = torch.from_numpy(ids).to(dev)
    out, status = q4.q4_gather_rows(c, s, idd, torch.bfloat16 if bf16 else torch.float32)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = out.view(torch.int16).cpu().numpy().view(np.uint16) if bf16 else out.cpu().numpy()
    if bf16:
        assert np.array_equal(got, ref), f"gather bf16 M={M} K={K}: {np.count_nonzero(got != ref)} differ"
    else:
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"gather f32 M={M} K={K}"
    _log(f"gather {dtype_name} M={M} K={K} n={n}: bit-exact")


@pytest.mark.parametrize("dtype_name", ["f32", "bf16"])
@pytest.mark.parametrize("M,K,n", GATHER_SHAPES)
def test_gather_rows_bit_exact(env, M, K, n, dtype_name):
    _gather_case(env, M, K, n, 7000 + M + K + n, dtype_name)


def test_gather_rows_bf16_ties(env):
    """Rows of +s, -s and 0 with s an exact bf16 midpoint (the fp32 product
    is exact, so the tie is decided by the even rule alone)."""
    torch, q4, dev = env
    K = 128
    svals = [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 2 + 2.0 ** -7, 0.5 + 3 * 2.0 ** -9]
    W = np.zeros((len(svals), K), np.float32)
    for r, sv in enumerate(svals):
        W[r, 0::3] = sv
        W[r, 1::3] = -sv
    codes, scales, _ = oracle.pack(W)
    ids = np.array([3, 2, 1, 0, 0], np.int32)
    ref, _ = oracle.gather_rows(codes, scales, len(svals), K, ids, bf16=True)
    c, s = _upload_packed(env, codes, scales)
    out, status = q4.q4_gather_rows(c, s, torch.from_numpy(ids).to(dev), torch.bfloat16)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), ref)


@pytest.mark.parametrize("dtype_name", ["f32", "bf16"])
def test_gather_rows_refuses_bad_ids(env, dtype_name):
    torch, q4, dev = env
    bf16 = dtype_name == "bf16"
    M, K = 50, 2048
    codes, scales, _ = oracle.pack(wl.weights(M, K, 7100, std=0.5))
    ids = np.array([4, -1, M, 49, 2 ** 31 - 1, 0], np.int32)
    ref, flags = oracle.gather_rows(codes, scales, M, K, ids, bf16=bf16)
    assert flags == oracle.GATHER_BAD_ID
    c, s = _upload_packed(env, codes, scales)
    dt = torch.bfloat16 if bf16 else torch.float32
    out = torch.full((len(ids), K), float("nan"), dtype=dt, device=dev)
    sentinel = out.clone()
    out, status = q4.q4_gather_rows(c, s, torch.from_numpy(ids).to(dev), dt, out)
    torch.cuda.synchronize()
    assert int(status.item()) == q4.Q4_GATHER_BAD_ID
    # every row, refused ones (zeros) included, equals the oracle's bits
    got = out.view(torch.int16).cpu().numpy().view(np.uint16) if bf16 else out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, ref.view(np.uint16 if bf16 else np.uint32))
    assert not np.any(got[[1, 2, 4]]), "a refused row is not zeros"
    del sentinel
    # the next good call clears the flag; n == 0 clears it too
    status.fill_(77)
    q4.q4_gather_rows(c, s, torch.from_numpy(ids[[0, 3]]).to(dev), dt, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    status.fill_(77)
    q4.q4_gather_rows(c, s, torch.empty(0, dtype=torch.int32, device=dev), dt, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0


def test_gather_rows_tied_lm_head_full_size(env):
    """The tied embedding: rows of the full lm_head matrix (151936 x 2048),
    packed by the oracle, gathered for a 32-token chunk and one token."""
    torch, q4, dev = env
    cfg = wl.CONFIGS["lm_head"]
    M, K = cfg["M"], cfg["K"]
    W = wl.weights(M, K, cfg["seed"])
    codes, scales, st = oracle.pack(W, threads=min(16, os.cpu_count() or 1))
    assert st == 0
    del W
    c, s = _upload_packed(env, codes, scales)
    rng = np.random.default_rng(7200)
    for n in (32, 1):
        ids = rng.integers(0, M, n).astype(np.int32)
        ids[0] = M - 1
        for bf16 in (False, True):
            ref, _ = oracle.gather_rows(codes, scales, M, K, ids, bf16=bf16)
            out, status = q4.q4_gather_rows(c, s, torch.from_numpy(ids).to(dev),
                                            torch.bfloat16 if bf16 else torch.float32)
            torch.cuda.synchronize()
            assert int(status.item()) == 0
            got = out.view(torch.int16).cpu().numpy().view(np.uint16) if bf16 else out.cpu().numpy().view(np.uint32)
            assert np.array_equal(got, ref.view(np.uint16 if bf16 else np.uint32)), f"lm_head gather n={n} bf16={bf16}"
    _log("gather lm_head 151936x2048: bit-exact for n=32 and n=1, fp32 and bf16")


# ---------------------------------------------------------------------------
# Affine format: q4_pack_affine (bit-exact) and q4_gemv_affine
# ---------------------------------------------------------------------------

def _affine_upload(env, codes, scales, zeros):
    torch, q4, dev = env
    c, s = _upload_packed(env, codes, scales)
    z = cases.to_dev(zeros.view(np.float16), torch, dev)
    return c, s, z


@pytest.mark.parametrize("M,K", [(1, 64), (17, 192), (256, 512), (5, 4096), (33, 11008)])
def test_affine_pack_bit_exact(env, M, K):
    torch, q4, dev = env
    W = wl.weights(M, K, 8000 + M + K, std=0.6)
    W[:, :64] += np.float32(0.7)        # blocks off zero
    if M > 2:
        W[1, 64:128] = 0.0 if K > 64 else W[1, 64:128]
        W[2, :64] = np.float32(-0.3)    # constant negative block
    c_ref, s_ref, z_ref, st_ref = oracle.pack_affine(W)
    codes, scales, zeros, status = q4.q4_pack_affine(cases.to_dev(W, torch, dev))
    torch.cuda.synchronize()
    assert int(status.item()) == st_ref == 0
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.view(torch.int16).cpu().numpy().view(np.uint16), s_ref)
    assert np.array_equal(zeros.view(torch.int16).cpu().numpy().view(np.uint16), z_ref)


def test_affine_pack_exact_ties_and_flags(env):
    torch, q4, dev = env
    W = np.zeros((3, 128), np.float32)
    W[0, :5] = [0.9375, -0.9375, 0.0625, -0.0625, 0.1875]   # s = 0.125, z = 7.5 -> 7, midpoint codes
    W[1, 64:70] = [1e-30, -1e-30, 3e-8, 0, 0, 0]              # below the fp16 range: s == 0
    W[2, 0], W[2, 1] = 4.0e5, -4.0e5                          # large but finite scale
    c_ref, s_ref, z_ref, st = oracle.pack_affine(W)
    assert st == 0
    codes, scales, zeros, status = q4.q4_pack_affine(cases.to_dev(W, torch, dev))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.view(torch.int16).cpu().numpy().view(np.uint16), s_ref)
    assert np.array_equal(zeros.view(torch.int16).cpu().numpy().view(np.uint16), z_ref)
    for bad, flag in ((np.nan, q4.Q4_PACK_NONFINITE), (6.0e5, q4.Q4_PACK_OVERFLOW)):
        Wb = W.copy()
        Wb[1, 3] = bad
        if flag == q4.Q4_PACK_OVERFLOW:
            Wb[1, 4] = -6.0e5
        _, _, _, st_b = oracle.pack_affine(Wb)
        assert st_b == flag
        _, _, _, sb = q4.q4_pack_affine(cases.to_dev(Wb, torch, dev))
        torch.cuda.synchronize()
        assert int(sb.item()) == flag


AFFINE_GEMV_SHAPES = [(1, 64), (7, 128), (1000, 1024), (4097, 2048), (40001, 64), (300, 2112), (65, 4096),
                      (129, 4160), (2048, 11008), (4101, 16448), (3, 32768), (2, 131072)]


@pytest.mark.parametrize("M,K", AFFINE_GEMV_SHAPES)
def test_affine_gemv_parity(env, M, K):
    torch, q4, dev = env
    seed = 8100 + M + K
    W = wl.weights(M, K, seed, std=0.5) + np.float32(0.05)
    x = wl.activation(K, seed, "normal")
    codes, scales, zeros, st = oracle.pack_affine(W)
    assert st == 0
    y_ref, S = oracle.gemv_affine(codes, scales, zeros, M, K, x)
    c, s, z = _affine_upload(env, codes, scales, zeros)
    y = q4.q4_gemv_affine(c, s, z, _x_dev(env, x))
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), y_ref, S, f"affine gemv M={M} K={K}")


def test_affine_full_size_gateup(env):
    """The gate/up shape (22016 x 2048): GPU pack bit-exact with the oracle,
    then the GEMV on every row against the oracle."""
    torch, q4, dev = env
    c_cfg = wl.CONFIGS["gateup"]
    M, K = c_cfg["M"], c_cfg["K"]
    W = wl.weights(M, K, c_cfg["seed"])
    x = wl.activation(K, c_cfg["seed"], c_cfg["x"])
    threads = min(16, os.cpu_count() or 1)
    c_ref, s_ref, z_ref, st = oracle.pack_affine(W, threads=threads)
    assert st == 0
    codes, scales, zeros, status = q4.q4_pack_affine(cases.to_dev(W, torch, dev))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.view(torch.int16).cpu().numpy().view(np.uint16), s_ref)
    assert np.array_equal(zeros.view(torch.int16).cpu().numpy().view(np.uint16), z_ref)
    y = q4.q4_gemv_affine(codes, scales, zeros, _x_dev(env, x))
    torch.cuda.synchronize()
    y_ref, S = oracle.gemv_affine(c_ref, s_ref, z_ref, M, K, x, threads=threads)
    _check(y.cpu().numpy(), y_ref, S, "affine gemv gate/up 22016x2048")


# ---------------------------------------------------------------------------
# NVFP4-style format: q4_pack_nvfp4 (bit-exact) and q4_gemv_nvfp4
# ---------------------------------------------------------------------------

def _nvfp4_gpu_pack(env, W):
    torch, q4, dev = env
    codes, scales, ts, status = q4.q4_pack_nvfp4(cases.to_dev(W, torch, dev))
    torch.cuda.synchronize()
    return codes, scales, ts, int(status.item())


def _nvfp4_check_pack(env, W):
    c_ref, s_ref, ts_ref, st_ref = oracle.pack_nvfp4(W)
    codes, scales, ts, st = _nvfp4_gpu_pack(env, W)
    assert st == st_ref == 0
    assert np.float32(ts.item()).view(np.uint32) == np.float32(ts_ref).view(np.uint32)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    return c_ref, s_ref, ts_ref


@pytest.mark.parametrize("M,K", [(1, 64), (17, 192), (256, 512), (5, 4096), (33, 11008)])
def test_nvfp4_pack_bit_exact(env, M, K):
    W = wl.weights(M, K, 9000 + M + K, std=0.5)
    if M > 2:
        W[1, 16:32] *= 1e-4      # subnormal E4M3 block scale
        W[2, 32:48] = 0.0        # zero block
        W[0, 5] = -0.0
    _nvfp4_check_pack(env, W)


def test_nvfp4_pack_ties_and_flags(env):
    torch, q4, dev = env
    W = np.zeros((2, 64), np.float32)
    W[0, 0] = 2688.0
    W[0, 16:32] = [6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -5, 0.5, 3, 0, -6, 4, 1.5]
    W[0, 32:34] = [6.375, 1.0]
    W[1, 0:16] = 1e-6            # tiny against the tensor scale: scale 0 or subnormal
    _nvfp4_check_pack(env, W)
    _nvfp4_check_pack(env, np.zeros((3, 128), np.float32))  # s == 0
    Wb = W.copy()
    Wb[1, 40] = np.nan
    _, _, _, st = _nvfp4_gpu_pack(env, Wb)
    assert st == q4.Q4_PACK_NONFINITE == oracle.pack_nvfp4(Wb)[3]


NVFP4_GEMV_SHAPES = [(1, 64), (7, 128), (1000, 1024), (4097, 2048), (40001, 64), (300, 2112), (65, 4096),
                     (129, 4160), (2048, 11008), (4101, 16448), (3, 32768), (2, 131072)]


@pytest.mark.parametrize("M,K", NVFP4_GEMV_SHAPES)
def test_nvfp4_gemv_parity(env, M, K):
    torch, q4, dev = env
    seed = 9100 + M + K
    W = wl.weights(M, K, seed, std=0.5)
    if M > 3:
        W[3, :64] *= 1e-4                 # subnormal block scales in the product
    x = wl.activation(K, seed, "normal")
    codes, scales, ts, st = oracle.pack_nvfp4(W)
    assert st == 0
    y_ref, S = oracle.gemv_nvfp4(codes, scales, ts, M, K, x)
    c = cases.to_dev(codes, torch, dev)
    s = cases.to_dev(scales, torch, dev)
    t = torch.tensor([ts], dtype=torch.float32, device=dev)
    y = q4.q4_gemv_nvfp4(c, s, t, _x_dev(env, x))
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), y_ref, S, f"nvfp4 gemv M={M} K={K}")


def test_nvfp4_full_size_gateup(env):
    """The gate/up shape: GPU pack bit-exact with the oracle, then the GEMV on
    every row (reading the tensor scale the pack wrote) against the oracle."""
    torch, q4, dev = env
    c_cfg = wl.CONFIGS["gateup"]
    M, K = c_cfg["M"], c_cfg["K"]
    W = wl.weights(M, K, c_cfg["seed"])
    x = wl.activation(K, c_cfg["seed"], c_cfg["x"])
    threads = min(16, os.cpu_count() or 1)
    c_ref, s_ref, ts_ref, st = oracle.pack_nvfp4(W, threads=threads)
    assert st == 0
    codes, scales, ts, st_g = _nvfp4_gpu_pack(env, W)
    assert st_g == 0 and ts.item() == ts_ref
    assert np.array_equal(codes.cpu().numpy(), c_ref) and np.array_equal(scales.cpu().numpy(), s_ref)
    y = q4.q4_gemv_nvfp4(codes, scales, ts, _x_dev(env, x))
    torch.cuda.synchronize()
    y_ref, S = oracle.gemv_nvfp4(c_ref, s_ref, ts_ref, M, K, x, threads=threads)
    _check(y.cpu().numpy(), y_ref, S, "nvfp4 gemv gate/up 22016x2048")


# ---------------------------------------------------------------------------
# int8 activations: q4_quantize_x8 (bit-exact) and q4_gemv_affine_x8
# ---------------------------------------------------------------------------

def _x8_dev(env, q1, q2, d):
    torch, q4, dev = env
    t1 = cases.to_dev(q1, torch, dev)
    t2 = cases.to_dev(q2, torch, dev) if q2 is not None else None
    return t1, t2, cases.to_dev(d, torch, dev)


@pytest.mark.parametrize("words", [1, 2])
@pytest.mark.parametrize("K,recipe", [(64, "normal"), (2048, "unit_rms"), (11008, "swiglu"), (131072, "normal")])
def test_quantize_x8_bit_exact(env, K, recipe, words):
    torch, q4, dev = env
    x = wl.activation(K, 9500 + K, recipe)
    if K >= 128:
        x[64:96] = 0                                   # a zero block
        x[96:128] = wl.bf16_rne_bits(np.full(32, 1e-30))  # a block of tiny values
        x[32:38] = wl.bf16_rne_bits(np.array([127.0, 2.5, 3.5, -2.5, 0.5, 0.50390625]))
        x[38:64] = 0
    q1r, q2r, dr = oracle.quantize_x8(x, words)
    q1, q2, d = q4.q4_quantize_x8(_x_dev(env, x), words)
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy().view(np.uint32), dr.view(np.uint32))
    assert np.array_equal(q1.cpu().numpy(), q1r)
    if words == 2:
        assert np.array_equal(q2.cpu().numpy(), q2r)


X8_GEMV_SHAPES = [(1, 64), (7, 128), (1000, 1024), (4097, 2048), (40001, 64), (300, 2112), (65, 4096),
                  (129, 4160), (2048, 11008), (4101, 16448), (3, 32768), (2, 131072)]


@pytest.mark.parametrize("words", [1, 2])
@pytest.mark.parametrize("M,K", X8_GEMV_SHAPES)
def test_affine_x8_gemv_parity(env, M, K, words):
    torch, q4, dev = env
    seed = 9600 + M + K
    W = wl.weights(M, K, seed, std=0.5) + np.float32(0.05)
    x = wl.activation(K, seed, "normal")
    codes, scales, zeros, st = oracle.pack_affine(W)
    assert st == 0
    q1, q2, d = oracle.quantize_x8(x, words)
    y_ref, S = oracle.gemv_affine_x8(codes, scales, zeros, M, K, q1, q2, d)
    c, s, z = _affine_upload(env, codes, scales, zeros)
    t1, t2, td = _x8_dev(env, q1, q2, d)
    y = q4.q4_gemv_affine_x8(c, s, z, t1, t2, td)
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), y_ref, S, f"affine x8 ({words} word) gemv M={M} K={K}")


# The affine format reads a tile's scales and zero points with one dword load
# each per lane when both planes are dword-aligned (an even number a row),
# else one 2-byte load per row each; a 2 mod 4 zero-point plane takes the
# second path, in every launch shape of one chunk a lane.
@pytest.mark.parametrize("shift", [0, 1])
@pytest.mark.parametrize("M,K", [(1001, 1024), (20011, 2048), (2053, 11008)])
def test_affine_zero_point_plane_alignment(env, M, K, shift):
    torch, q4, dev = env
    seed = 9900 + M + K
    W = wl.weights(M, K, seed, std=0.5) + np.float32(0.05)
    x = wl.activation(K, seed, "normal")
    codes, scales, zeros, st = oracle.pack_affine(W)
    assert st == 0
    c, s, _ = _affine_upload(env, codes, scales, zeros)
    z = _scales_at(env, zeros, shift)
    assert z.data_ptr() % 4 == 2 * shift
    y_ref, S = oracle.gemv_affine(codes, scales, zeros, M, K, x)
    y = q4.q4_gemv_affine(c, s, z, _x_dev(env, x))
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), y_ref, S, f"affine gemv M={M} K={K} zeros +{2 * shift} B")
    q1, q2, d = oracle.quantize_x8(x, 2)
    y8_ref, S8 = oracle.gemv_affine_x8(codes, scales, zeros, M, K, q1, q2, d)
    t1, t2, td = _x8_dev(env, q1, q2, d)
    y8 = q4.q4_gemv_affine_x8(c, s, z, t1, t2, td)
    torch.cuda.synchronize()
    _check(y8.cpu().numpy(), y8_ref, S8, f"affine x8 gemv M={M} K={K} zeros +{2 * shift} B")


def test_affine_x8_chain_full_size_down(env):
    """The down shape (2048 x 11008, SwiGLU-like x): GPU pack, GPU quantise
    and the GEMV against the oracle's pack, quantise and GEMV; the bf16
    product and the two-word product stay within the restated bound of
    each other (|x - xq| <= d / 256)."""
    torch, q4, dev = env
    c_cfg = wl.CONFIGS["down"]
    M, K = c_cfg["M"], c_cfg["K"]
    W = wl.weights(M, K, c_cfg["seed"])
    x = wl.activation(K, c_cfg["seed"], c_cfg["x"])
    codes, scales, zeros, st = q4.q4_pack_affine(cases.to_dev(W, torch, dev))
    c_ref, s_ref, z_ref, _ = oracle.pack_affine(W, threads=min(16, os.cpu_count() or 1))
    for words in (2, 1):
        q1, q2, d = q4.q4_quantize_x8(_x_dev(env, x), words)
        y = q4.q4_gemv_affine_x8(codes, scales, zeros, q1, q2, d)
        torch.cuda.synchronize()
        r1, r2, rd = oracle.quantize_x8(x, words)
        y_ref, S = oracle.gemv_affine_x8(c_ref, s_ref, z_ref, M, K, r1, r2, rd, threads=min(16, os.cpu_count() or 1))
        _check(y.cpu().numpy(), y_ref, S, f"affine x8 chain down ({words} word)")
    # restated against the bf16 product: |y(xq) - y(x)| <= sum |What| |x - xq|
    yb, _ = oracle.gemv_affine(c_ref, s_ref, z_ref, M, K, x)
    r1, r2, rd = oracle.quantize_x8(x, 2)
    xq = oracle.dequantize_x8(r1, r2, rd)
    xv = wl.bf16_bits_to_f32(x).astype(np.float64)
    What = oracle.dequant_affine(c_ref, s_ref, z_ref, M, K)
    bound = np.abs(What) @ np.abs(xq - xv)
    y2, _ = oracle.gemv_affine_x8(c_ref, s_ref, z_ref, M, K, r1, r2, rd)
    assert np.all(np.abs(y2 - yb) <= bound * (1 + 1e-9) + 1e-12)


def test_graph_capture_other_entry_points(env):
    """Gather, affine, NVFP4-style (GEMV, prefill on 4-row and 16-row
    tiles, fused SwiGLU and bias forms), int8 quantisation and int8 GEMV
    captured in one graph; every replay (with eager work in between) equals
    eager."""
    torch, q4, dev = env
    M, K = 3000, 2048
    W = wl.weights(M, K, 7300)
    Wd = cases.to_dev(W, torch, dev)
    xd = _x_dev(env, wl.activation(K, 7300, "unit_rms"))
    X4 = cases.to_dev(wl.activations(4, K, 7301, "unit_rms").view(np.int16), torch, dev).view(torch.bfloat16)
    X17 = cases.to_dev(wl.activations(17, K, 7302, "unit_rms").view(np.int16), torch, dev).view(torch.bfloat16)
    codes, scales, _ = oracle.pack(W)
    c, s = _upload_packed(env, codes, scales)
    ac, asc, az, _ = q4.q4_pack_affine(Wd)
    nc, ns, nt, _ = q4.q4_pack_nvfp4(Wd)
    torch.cuda.synchronize()
    ids = torch.tensor([5, 0, M - 1, 17], dtype=torch.int32, device=dev)
    h = M // 2
    bias = torch.linspace(-1.0, 1.0, M, device=dev)

    def run(outs=None):
        o = outs or {}
        g, st = q4.q4_gather_rows(c, s, ids, torch.bfloat16, o.get("g"), o.get("gs"))
        ya = q4.q4_gemv_affine(ac, asc, az, xd, o.get("ya"))
        yn = q4.q4_gemv_nvfp4(nc, ns, nt, xd, o.get("yn"))
        q1, q2, d = q4.q4_quantize_x8(xd, 2, o.get("q1"), o.get("q2"), o.get("d"))
        y8 = q4.q4_gemv_affine_x8(ac, asc, az, q1, q2, d, o.get("y8"))
        Ya4 = q4.q4_gemm_smalln_affine(ac, asc, az, X4, o.get("Ya4"))
        Yn4 = q4.q4_gemm_smalln_nvfp4(nc, ns, nt, X4, o.get("Yn4"))
        Ya17 = q4.q4_gemm_smalln_affine(ac, asc, az, X17, o.get("Ya17"))
        fa = q4.q4_gemv_fused_affine([(ac[:h], asc[:h], az[:h], None), (ac[h:], asc[h:], az[h:], None)], xd,
                                     "swiglu", [o["fa"]] if "fa" in o else None)[0]
        fn = q4.q4_gemv_fused_nvfp4([(nc, ns, nt, bias)], xd, "separate", [o["fn"]] if "fn" in o else None)[0]
        return {"g": g, "gs": st, "ya": ya, "yn": yn, "q1": q1, "q2": q2, "d": d, "y8": y8, "Ya4": Ya4,
                "Yn4": Yn4, "Ya17": Ya17, "fa": fa, "fn": fn}

    eager = {k: v.clone() for k, v in run().items()}
    torch.cuda.synchronize()
    outs = {k: torch.empty_like(v) for k, v in eager.items()}
    gr = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        with torch.cuda.graph(gr, stream=stream):
            run(outs)
    torch.cuda.synchronize()
    for rep in range(3):
        for v in outs.values():
            v.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(outs[k].view(torch.uint8), eager[k].view(torch.uint8)), f"replay {rep}: {k} differs"
        run()  # eager work between replays
        torch.cuda.synchronize()
