"""The C ABI without a GPU: the library loads, exports every entry point that
include/q4.h declares, and refuses bad arguments on the host before any
launch (golang.design accel/tensor conventions: validate everything first,
refuse rather than clamp).  The pointers used here are never dereferenced:
each call fails a host-side check first.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")


@pytest.fixture(scope="module")
def q4():
    import bit_weight_gemv_amd as q4
    if not os.path.exists(q4.LIB_PATH):
        from bit_weight_gemv_amd import build
        build.build()
    return q4


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("q4_pack", "q4_unpack_canonical", "q4_gemv", "q4_gemm_smalln", "q4_gemv_fused",
              "q4_gather_rows", "q4_pack_affine", "q4_gemv_affine", "q4_pack_nvfp4", "q4_gemv_nvfp4",
              "q4_quantize_x8", "q4_gemv_affine_x8", "q4_gemm_smalln_affine", "q4_gemm_smalln_nvfp4",
              "q4_gemv_fused_affine", "q4_gemv_fused_nvfp4", "q4_codebook", "q4_codes_bytes",
              "q4_scales_bytes", "q4_status_string", "q4_gemm_smalln_ws_bytes", "q4_gemm_smalln_ws",
              "q4_gemm_smalln_noalloc", "q4_gemm_smalln_affine_ws",
              "q4_gemm_smalln_nvfp4_ws"):
        assert n in names


def test_library_exports_every_declared_symbol(q4):
    L = q4.lib()
    for name in _declared_functions():
        assert hasattr(L, name), f"libq4.so does not export {name}"
    assert set(_declared_functions()) == set(q4.EXPORTED)


def test_codebook_is_the_oracles(q4, oracle_mod):
    lib_levels = np.array(q4.codebook(), np.float32)
    assert np.array_equal(lib_levels.view(np.uint32), oracle_mod.codebook_f32().view(np.uint32))


def test_sizes(q4):
    assert q4.codes_bytes(151936, 2048) == 151936 * 1024
    assert q4.scales_bytes(151936, 2048) == 151936 * 32 * 2
    assert q4.codes_bytes(3, 64) == 96 and q4.scales_bytes(3, 64) == 6
    assert q4.codes_bytes(0, 64) == 0
    assert q4.codes_bytes(4, 100) == 0 and q4.scales_bytes(-1, 64) == 0
    assert q4.codes_bytes(1, q4.Q4_MAX_K + 64) == 0


def test_status_strings(q4):
    for s in range(7):
        assert q4.status_string(s).startswith("Q4_")
    assert "unknown" in q4.status_string(99)


A = 0x10000000  # fake, aligned, never dereferenced
B = 0x20000000
C = 0x30000000
D = 0x40000000


def _gemv(q4, codes, scales, M, K, x, y):
    return q4.lib().q4_gemv(codes, scales, M, K, x, y, None)


def _gemm(q4, codes, scales, M, K, X, N, Y):
    return q4.lib().q4_gemm_smalln(codes, scales, M, K, X, N, Y, None)


def _pack(q4, W, M, K, codes, scales, status):
    return q4.lib().q4_pack(W, M, K, codes, scales, status, None)


def test_gemv_shape_errors(q4):
    for M, K in [(-1, 64), (4, 0), (4, 63), (4, 100), (4, -64), (4, q4.Q4_MAX_K + 64), (1 << 60, 1024)]:
        assert _gemv(q4, A, B, M, K, C, D) == q4.Q4_ERR_SHAPE, (M, K)


def test_gemv_empty_is_noop(q4):
    assert _gemv(q4, None, None, 0, 64, None, None) == q4.Q4_OK


def test_gemv_null_and_alignment(q4):
    M, K = 16, 128
    assert _gemv(q4, None, B, M, K, C, D) == q4.Q4_ERR_NULL
    assert _gemv(q4, A, None, M, K, C, D) == q4.Q4_ERR_NULL
    assert _gemv(q4, A, B, M, K, None, D) == q4.Q4_ERR_NULL
    assert _gemv(q4, A, B, M, K, C, None) == q4.Q4_ERR_NULL
    assert _gemv(q4, A + 8, B, M, K, C, D) == q4.Q4_ERR_ALIGN
    assert _gemv(q4, A, B + 1, M, K, C, D) == q4.Q4_ERR_ALIGN
    assert _gemv(q4, A, B, M, K, C + 2, D) == q4.Q4_ERR_ALIGN
    assert _gemv(q4, A, B, M, K, C, D + 2) == q4.Q4_ERR_ALIGN


def test_gemv_overlap(q4):
    M, K = 16, 128  # codes 1024 B, scales 64 B, x 256 B, y 64 B
    assert _gemv(q4, A, B, M, K, C, A + 1020) == q4.Q4_ERR_OVERLAP   # y over codes tail
    assert _gemv(q4, A, B, M, K, C, B) == q4.Q4_ERR_OVERLAP          # y on scales
    assert _gemv(q4, A, B, M, K, C, C + 252) == q4.Q4_ERR_OVERLAP    # y over x tail
    # every call here must fail a host check: a call that passed them all
    # would launch on fake pointers
    assert _gemv(q4, A, B, M, K, C + 2, A + 1024) == q4.Q4_ERR_ALIGN


def test_gemm_shape_errors(q4):
    assert _gemm(q4, A, B, 16, 128, C, 33, D) == q4.Q4_ERR_SHAPE
    assert _gemm(q4, A, B, 16, 128, C, -1, D) == q4.Q4_ERR_SHAPE
    assert _gemm(q4, A, B, 16, 96, C, 4, D) == q4.Q4_ERR_SHAPE
    assert _gemm(q4, None, None, 16, 128, None, 0, None) == q4.Q4_OK
    assert _gemm(q4, None, None, 0, 128, None, 5, None) == q4.Q4_OK


def test_gemm_null_alignment_overlap(q4):
    M, K, N = 16, 128, 4
    assert _gemm(q4, A, B, M, K, None, N, D) == q4.Q4_ERR_NULL
    assert _gemm(q4, A, B, M, K, C + 8, N, D) == q4.Q4_ERR_ALIGN
    assert _gemm(q4, A, B, M, K, C, N, D + 1) == q4.Q4_ERR_ALIGN
    assert _gemm(q4, A, B, M, K, C, N, C + 1020) == q4.Q4_ERR_OVERLAP  # Y over X's last word (X is 1 KB)


def _gemm_ws(q4, codes, scales, M, K, X, N, Y, ws, nb):
    return q4.lib().q4_gemm_smalln_ws(codes, scales, M, K, X, N, Y, ws, nb, None)


def test_gemm_ws_bytes(q4):
    """Scratch is asked for exactly where the long-row split runs: chunks of
    2..32 tokens on rows longer than 2048 weights, except those the grouped
    GEMV takes (2 and 3 tokens; 4 tokens from rows of 8192 weights); its
    size is ranges x N x M fp32 with ranges of at most 2048 weights."""
    nb = q4.q4_gemm_smalln_ws_bytes
    assert nb(2048, 11008, 32) == 6 * 32 * 2048 * 4  # 43 slices of 256: 6 ranges
    assert nb(2048, 11008, 5) == 6 * 5 * 2048 * 4
    assert nb(5120, 5120, 4) == 3 * 4 * 5120 * 4      # 4 tokens on rows of 5120: the split
    assert nb(2048, 11008, 4) == 0                    # the grouped GEMV
    assert nb(2048, 11008, 3) == 0 and nb(2048, 11008, 2) == 0 and nb(2048, 11008, 1) == 0
    assert nb(11008, 2048, 32) == 0                   # rows of 2048: one range
    assert nb(1, 2112, 5) == 2 * 5 * 4                # 9 slices: two ranges
    assert nb(3, 131072, 32) == 64 * 32 * 3 * 4
    assert nb(0, 11008, 8) == 0 and nb(16, 11008, 33) == 0 and nb(16, 100, 8) == 0


def test_gemm_ws_errors(q4):
    M, K, N = 16, 11008, 8              # codes 88064 B, scales 5504 B, X 176128 B, Y 512 B
    need = q4.q4_gemm_smalln_ws_bytes(M, K, N)
    assert need == 6 * N * M * 4
    E = 0x50000000
    assert _gemm_ws(q4, A, B, M, K, C, N, D, None, 0) == q4.Q4_ERR_WORKSPACE
    assert _gemm_ws(q4, A, B, M, K, C, N, D, E, need - 4) == q4.Q4_ERR_WORKSPACE
    assert _gemm_ws(q4, A, B, M, K, C, N, D, E + 4, need) == q4.Q4_ERR_ALIGN
    assert _gemm_ws(q4, A, B, M, K, C, N, D, D + 256, need) == q4.Q4_ERR_OVERLAP   # over Y's tail
    assert _gemm_ws(q4, A, B, M, K, C, N, D, C + 1024, need) == q4.Q4_ERR_OVERLAP  # over X
    assert _gemm_ws(q4, A, B, M, K, C, 33, D, E, need) == q4.Q4_ERR_SHAPE
    assert _gemm_ws(q4, A, B, M, K, None, N, D, E, need) == q4.Q4_ERR_NULL
    assert _gemm_ws(q4, None, None, 0, K, None, N, None, None, 0) == q4.Q4_OK


def test_gemm_formats_ws_checks(q4):
    """The affine and NVFP4-style *_ws products take scratch on the same
    chunks as q4_gemm_smalln_ws, sized by q4_gemm_smalln_ws_bytes, and check
    it the same way."""
    nb = q4.q4_gemm_smalln_ws_bytes
    L = q4.lib()
    M, K, N = 16, 11008, 8
    need = nb(M, K, N)
    E = 0x50000000
    Z = 0x60000000
    aff = lambda ws, n_b, zeros=Z: L.q4_gemm_smalln_affine_ws(A, B, zeros, M, K, C, N, D, ws, n_b, None)
    nv = lambda ws, n_b: L.q4_gemm_smalln_nvfp4_ws(A, B, Z, M, K, C, N, D, ws, n_b, None)
    assert aff(None, 0) == q4.Q4_ERR_WORKSPACE and nv(None, 0) == q4.Q4_ERR_WORKSPACE
    assert aff(E, need - 4) == q4.Q4_ERR_WORKSPACE and nv(E, need - 4) == q4.Q4_ERR_WORKSPACE
    assert aff(E + 4, need) == q4.Q4_ERR_ALIGN and nv(E + 4, need) == q4.Q4_ERR_ALIGN
    assert aff(Z, need) == q4.Q4_ERR_OVERLAP          # over the zero points
    assert aff(E, need, zeros=None) == q4.Q4_ERR_NULL
    assert nv(C + 1024, need) == q4.Q4_ERR_OVERLAP     # over X


def test_gemm_noalloc_host_checks(q4):
    """The allocation-free entry point refuses, before any launch or device
    lookup, chunks whose partial sums exceed its fixed scratch, and the
    usual bad arguments."""
    L = q4.lib()
    M, K, N = 151936, 4096, 32       # two K ranges: 2 x 32 x 151936 x 4 bytes
    assert q4.q4_gemm_smalln_ws_bytes(M, K, N) > q4.Q4_NOALLOC_SCRATCH_BYTES
    big_codes, big_scales, big_x, big_y = 0x100000000, 0x200000000, 0x300000000, 0x400000000
    assert L.q4_gemm_smalln_noalloc(big_codes, big_scales, M, K, big_x, N, big_y, None) == q4.Q4_ERR_WORKSPACE
    assert q4.q4_gemm_smalln_ws_bytes(2048, 11008, 32) <= q4.Q4_NOALLOC_SCRATCH_BYTES
    assert L.q4_gemm_smalln_noalloc(A, B, 16, 11008, C, 33, D, None) == q4.Q4_ERR_SHAPE
    assert L.q4_gemm_smalln_noalloc(A, B, 16, 11008, None, 8, D, None) == q4.Q4_ERR_NULL
    assert L.q4_gemm_smalln_noalloc(A, B, 16, 11008, C + 8, 8, D, None) == q4.Q4_ERR_ALIGN
    assert L.q4_gemm_smalln_noalloc(A, B, 16, 11008, C, 8, C + 256, None) == q4.Q4_ERR_OVERLAP
    assert L.q4_gemm_smalln_noalloc(None, None, 0, 11008, None, 8, None, None) == q4.Q4_OK


def test_pack_errors(q4):
    assert _pack(q4, A, 4, 100, B, C, D) == q4.Q4_ERR_SHAPE
    assert _pack(q4, None, 4, 64, B, C, D) == q4.Q4_ERR_NULL
    assert _pack(q4, A, 4, 64, B, C, None) == q4.Q4_ERR_NULL
    assert _pack(q4, A + 4, 4, 64, B, C, D) == q4.Q4_ERR_ALIGN
    assert _pack(q4, A, 4, 64, B + 8, C, D) == q4.Q4_ERR_ALIGN
    assert _pack(q4, A, 4, 64, B, C + 1, D) == q4.Q4_ERR_ALIGN
    assert _pack(q4, A, 4, 64, B, C, D + 2) == q4.Q4_ERR_ALIGN
    assert _pack(q4, A, 4, 64, A + 512, C, D) == q4.Q4_ERR_OVERLAP  # codes inside W (1 KB)
    assert _pack(q4, A, 4, 64, B, B + 64, D) == q4.Q4_ERR_OVERLAP   # scales inside codes
    assert _pack(q4, A, 4, 64, B, C, C + 4) == q4.Q4_ERR_OVERLAP    # status inside scales


def _unpack(q4, codes, scales, M, K, co, so):
    return q4.lib().q4_unpack_canonical(codes, scales, M, K, co, so, None)


def test_unpack_errors(q4):
    M, K = 4, 128  # codes 256 B, scales 16 B
    assert _unpack(q4, A, B, 4, 100, C, D) == q4.Q4_ERR_SHAPE
    assert _unpack(q4, None, None, 0, 64, None, None) == q4.Q4_OK
    assert _unpack(q4, None, B, M, K, C, D) == q4.Q4_ERR_NULL
    assert _unpack(q4, A, B, M, K, C, None) == q4.Q4_ERR_NULL
    assert _unpack(q4, A + 8, B, M, K, C, D) == q4.Q4_ERR_ALIGN
    assert _unpack(q4, A, B, M, K, C + 8, D) == q4.Q4_ERR_ALIGN
    assert _unpack(q4, A, B, M, K, C, D + 1) == q4.Q4_ERR_ALIGN
    assert _unpack(q4, A, B, M, K, A + 128, D) == q4.Q4_ERR_OVERLAP   # codes_out inside codes
    assert _unpack(q4, A, B, M, K, C, B + 8) == q4.Q4_ERR_OVERLAP     # scales_out over scales
    assert _unpack(q4, A, B, M, K, C, C + 16) == q4.Q4_ERR_OVERLAP    # scales_out inside codes_out


def _fused(q4, ops, K, x, mode, ys, res=None):
    """ops: list of (codes, scales, M, bias) fake addresses; ys/res: lists."""
    arr = (q4.Operand * max(len(ops), 1))(*[q4.Operand(c, s, M, b) for c, s, M, b in ops])
    yp = (ctypes.c_void_p * max(len(ys), 1))(*ys) if ys is not None else None
    rp = (ctypes.c_void_p * max(len(res), 1))(*res) if res is not None else None
    return q4.lib().q4_gemv_fused(ctypes.cast(arr, ctypes.c_void_p) if ops else None, len(ops), K, x, mode,
                                  ctypes.cast(yp, ctypes.c_void_p) if yp is not None else None,
                                  ctypes.cast(rp, ctypes.c_void_p) if rp is not None else None, None)


E = 0x50000000
F = 0x60000000
G = 0x70000000


def test_fused_shape_and_mode_errors(q4):
    SEP, SWI = q4.Q4_FUSE_SEPARATE, q4.Q4_FUSE_SWIGLU
    op = (A, B, 16, 0)  # codes 1 KB at K=128, scales 64 B
    assert _fused(q4, [op], 128, C, 2, [D]) == q4.Q4_ERR_SHAPE               # unknown mode
    assert _fused(q4, [], 128, C, SEP, [D]) == q4.Q4_ERR_SHAPE                # no matrix
    assert _fused(q4, [op] * 5, 128, C, SEP, [D] * 5) == q4.Q4_ERR_SHAPE      # more than Q4_MAX_FUSED
    assert _fused(q4, [op] * 3, 128, C, SWI, [D]) == q4.Q4_ERR_SHAPE          # SwiGLU takes two
    assert _fused(q4, [op, (E, F, 8, 0)], 128, C, SWI, [D]) == q4.Q4_ERR_SHAPE  # unequal M
    assert _fused(q4, [op], q4.Q4_MAX_FUSED_K + 64, C, SEP, [D]) == q4.Q4_ERR_SHAPE
    assert _fused(q4, [op], 100, C, SEP, [D]) == q4.Q4_ERR_SHAPE
    assert _fused(q4, [(A, B, -1, 0)], 128, C, SEP, [D]) == q4.Q4_ERR_SHAPE
    assert _fused(q4, [(0, 0, 0, 0), (0, 0, 0, 0)], 128, 0, SEP, [0, 0]) == q4.Q4_OK  # nothing to do


def test_fused_null_and_alignment(q4):
    SEP = q4.Q4_FUSE_SEPARATE
    op = (A, B, 16, 0)
    assert _fused(q4, [op], 128, 0, SEP, [D]) == q4.Q4_ERR_NULL              # x
    assert _fused(q4, [op], 128, C, SEP, None) == q4.Q4_ERR_NULL             # y array
    assert _fused(q4, [op], 128, C, SEP, [0]) == q4.Q4_ERR_NULL              # y[0]
    assert _fused(q4, [(0, B, 16, 0)], 128, C, SEP, [D]) == q4.Q4_ERR_NULL   # codes
    assert _fused(q4, [op], 128, C + 8, SEP, [D]) == q4.Q4_ERR_ALIGN
    assert _fused(q4, [(A + 8, B, 16, 0)], 128, C, SEP, [D]) == q4.Q4_ERR_ALIGN
    assert _fused(q4, [(A, B + 1, 16, 0)], 128, C, SEP, [D]) == q4.Q4_ERR_ALIGN
    assert _fused(q4, [(A, B, 16, E + 2)], 128, C, SEP, [D]) == q4.Q4_ERR_ALIGN
    assert _fused(q4, [op], 128, C, SEP, [D + 2]) == q4.Q4_ERR_ALIGN
    assert _fused(q4, [op], 128, C, SEP, [D], [F + 2]) == q4.Q4_ERR_ALIGN


def test_fused_overlap(q4):
    SEP, SWI = q4.Q4_FUSE_SEPARATE, q4.Q4_FUSE_SWIGLU
    op = (A, B, 16, E)  # codes 1 KB, scales 64 B, bias 64 B; y 64 B
    assert _fused(q4, [op], 128, C, SEP, [A + 512]) == q4.Q4_ERR_OVERLAP       # y inside codes
    assert _fused(q4, [op], 128, C, SEP, [C + 200]) == q4.Q4_ERR_OVERLAP       # y over x's tail (256 B)
    assert _fused(q4, [op], 128, C, SEP, [E + 32]) == q4.Q4_ERR_OVERLAP        # y over the bias
    assert _fused(q4, [op, (F, G, 16, 0)], 128, C, SEP, [D, D + 32]) == q4.Q4_ERR_OVERLAP  # y0 over y1
    assert _fused(q4, [op], 128, C, SEP, [D], [D + 4]) == q4.Q4_ERR_OVERLAP    # residual shifted onto y
    assert _fused(q4, [op, (F, G, 16, 0)], 128, C, SEP, [D, D + 4096], [0, D + 16]) == q4.Q4_ERR_OVERLAP
    assert _fused(q4, [op, (F, G, 16, 0)], 128, C, SWI, [G + 16]) == q4.Q4_ERR_OVERLAP  # y over up scales


def _fused_fmt(q4, fmt, ops, K, x, mode, ys, res=None):
    """fmt "affine": ops (codes, scales, zeros, M, bias); "nvfp4": (codes,
    scales, tscale, M, bias); fake addresses."""
    st = q4.OperandAffine if fmt == "affine" else q4.OperandNvfp4
    fn = q4.lib().q4_gemv_fused_affine if fmt == "affine" else q4.lib().q4_gemv_fused_nvfp4
    arr = (st * max(len(ops), 1))(*[st(*op) for op in ops])
    yp = (ctypes.c_void_p * max(len(ys), 1))(*ys) if ys is not None else None
    rp = (ctypes.c_void_p * max(len(res), 1))(*res) if res is not None else None
    return fn(ctypes.cast(arr, ctypes.c_void_p) if ops else None, len(ops), K, x, mode,
              ctypes.cast(yp, ctypes.c_void_p) if yp is not None else None,
              ctypes.cast(rp, ctypes.c_void_p) if rp is not None else None, None)


def test_fused_formats_host_checks(q4):
    """The affine and NVFP4-style fused entry points: the shared checks, plus
    their own operands (zero points, E4M3 scales, tensor scale) as inputs."""
    SEP, SWI = q4.Q4_FUSE_SEPARATE, q4.Q4_FUSE_SWIGLU
    aop = (A, B, E, 16, 0)   # codes 1 KB at K=128, scales 64 B, zeros 64 B at E
    nop = (A, B, E, 16, 0)   # E4M3 scales 128 B at B, tensor scale at E
    for fmt, op in (("affine", aop), ("nvfp4", nop)):
        assert _fused_fmt(q4, fmt, [op], 128, C, 2, [D]) == q4.Q4_ERR_SHAPE
        assert _fused_fmt(q4, fmt, [op] * 3, 128, C, SWI, [D]) == q4.Q4_ERR_SHAPE
        assert _fused_fmt(q4, fmt, [op], 100, C, SEP, [D]) == q4.Q4_ERR_SHAPE
        assert _fused_fmt(q4, fmt, [], 128, C, SEP, [D]) == q4.Q4_ERR_SHAPE
        assert _fused_fmt(q4, fmt, [(0, 0, 0, 0, 0)], 128, 0, SEP, [0]) == q4.Q4_OK   # nothing to do
        assert _fused_fmt(q4, fmt, [op], 128, 0, SEP, [D]) == q4.Q4_ERR_NULL
        assert _fused_fmt(q4, fmt, [(A, B, 0, 16, 0)], 128, C, SEP, [D]) == q4.Q4_ERR_NULL  # zeros / tscale
        assert _fused_fmt(q4, fmt, [(A, B + 1, E, 16, 0)], 128, C, SEP, [D]) == q4.Q4_ERR_ALIGN
        assert _fused_fmt(q4, fmt, [op], 128, C, SEP, [D + 2]) == q4.Q4_ERR_ALIGN
        assert _fused_fmt(q4, fmt, [op], 128, C, SEP, [E]) == q4.Q4_ERR_OVERLAP      # y over zeros / tscale
        assert _fused_fmt(q4, fmt, [op], 128, C, SEP, [A + 512]) == q4.Q4_ERR_OVERLAP
    assert _fused_fmt(q4, "affine", [(A, B, E + 1, 16, 0)], 128, C, SEP, [D]) == q4.Q4_ERR_ALIGN
    assert _fused_fmt(q4, "nvfp4", [(A, B, E + 2, 16, 0)], 128, C, SEP, [D]) == q4.Q4_ERR_ALIGN
    # NVFP4-style scales are K / 16 bytes a row: y 64 B after the scales' start
    # overlaps them (it would not for fp16 scales of the same M).
    assert _fused_fmt(q4, "nvfp4", [nop], 128, C, SEP, [B + 64]) == q4.Q4_ERR_OVERLAP

    # every call above fails a host check; the exact-alias residual is legal
    # and is exercised on the GPU, not here


def _gather(q4, codes, scales, M, K, ids, n, out_type, out, status):
    return q4.lib().q4_gather_rows(codes, scales, M, K, ids, n, out_type, out, status, None)


def test_gather_errors(q4):
    F32, BF = q4.Q4_OUT_F32, q4.Q4_OUT_BF16
    # codes A (M=16, K=128: 1 KB), scales B (64 B), ids C (n=4: 16 B), out D, status E
    assert _gather(q4, A, B, 16, 100, C, 4, F32, D, E) == q4.Q4_ERR_SHAPE
    assert _gather(q4, A, B, -1, 128, C, 4, F32, D, E) == q4.Q4_ERR_SHAPE
    assert _gather(q4, A, B, 16, 128, C, -1, F32, D, E) == q4.Q4_ERR_SHAPE
    assert _gather(q4, A, B, 16, 128, C, 4, 2, D, E) == q4.Q4_ERR_SHAPE
    assert _gather(q4, A, B, 16, 128, C, 1 << 40, F32, D, E) == q4.Q4_ERR_SHAPE  # grid too large
    assert _gather(q4, A, B, 16, 128, C, 4, F32, D, 0) == q4.Q4_ERR_NULL
    assert _gather(q4, A, B, 16, 128, 0, 4, F32, D, E) == q4.Q4_ERR_NULL
    assert _gather(q4, A, B, 16, 128, C, 4, F32, 0, E) == q4.Q4_ERR_NULL
    assert _gather(q4, 0, B, 16, 128, C, 4, F32, D, E) == q4.Q4_ERR_NULL
    assert _gather(q4, A + 8, B, 16, 128, C, 4, F32, D, E) == q4.Q4_ERR_ALIGN
    assert _gather(q4, A, B + 1, 16, 128, C, 4, F32, D, E) == q4.Q4_ERR_ALIGN
    assert _gather(q4, A, B, 16, 128, C + 2, 4, F32, D, E) == q4.Q4_ERR_ALIGN
    assert _gather(q4, A, B, 16, 128, C, 4, BF, D + 8, E) == q4.Q4_ERR_ALIGN
    assert _gather(q4, A, B, 16, 128, C, 4, F32, D, E + 2) == q4.Q4_ERR_ALIGN
    assert _gather(q4, A, B, 16, 128, C, 4, F32, A + 512, E) == q4.Q4_ERR_OVERLAP   # out over codes
    assert _gather(q4, A, B, 16, 128, C, 4, F32, D, C + 4) == q4.Q4_ERR_OVERLAP     # status over ids
    assert _gather(q4, A, B, 16, 128, C, 4, BF, D, D + 1020) == q4.Q4_ERR_OVERLAP   # status in out (1 KB)
    assert _gather(q4, A, B, 16, 128, C, 4, F32, C - 2032, E) == q4.Q4_ERR_OVERLAP  # out's tail over ids
    # every call above fails a host check and launches nothing


def test_affine_errors(q4):
    L = q4.lib()
    # W A (M=16, K=128 fp32: 8 KB), codes B (1 KB), scales C (64 B), zeros D, status E
    assert L.q4_pack_affine(A, 16, 100, B, C, D, E, None) == q4.Q4_ERR_SHAPE
    assert L.q4_pack_affine(A, 16, 128, B, C, 0, E, None) == q4.Q4_ERR_NULL
    assert L.q4_pack_affine(A, 16, 128, B, C, D + 1, E, None) == q4.Q4_ERR_ALIGN
    assert L.q4_pack_affine(A, 16, 128, B, C, C + 32, E, None) == q4.Q4_ERR_OVERLAP   # zeros over scales
    assert L.q4_pack_affine(A, 16, 128, B, C, A + 4096, E, None) == q4.Q4_ERR_OVERLAP  # zeros inside W
    # gemv: codes A, scales B, zeros C, x D (256 B), y E (64 B)
    assert L.q4_gemv_affine(A, B, C, 16, 100, D, E, None) == q4.Q4_ERR_SHAPE
    assert L.q4_gemv_affine(A, B, C, 0, 128, 0, 0, None) == q4.Q4_OK
    assert L.q4_gemv_affine(A, B, 0, 16, 128, D, E, None) == q4.Q4_ERR_NULL
    assert L.q4_gemv_affine(A, B, C + 1, 16, 128, D, E, None) == q4.Q4_ERR_ALIGN
    assert L.q4_gemv_affine(A, B, C, 16, 128, D, C + 16, None) == q4.Q4_ERR_OVERLAP  # y over zeros
    # every call above fails a host check and launches nothing


def test_nvfp4_errors(q4):
    L = q4.lib()
    # W A (M=16, K=128 fp32: 8 KB), codes B (1 KB), scales C (128 B), tscale D, status E
    assert L.q4_pack_nvfp4(A, 16, 100, B, C, D, E, None) == q4.Q4_ERR_SHAPE
    assert L.q4_pack_nvfp4(A, 16, 128, B, C, 0, E, None) == q4.Q4_ERR_NULL
    assert L.q4_pack_nvfp4(A, 16, 128, B, C + 1, D, E, None) == q4.Q4_ERR_ALIGN
    assert L.q4_pack_nvfp4(A, 16, 128, B, C, D + 2, E, None) == q4.Q4_ERR_ALIGN
    assert L.q4_pack_nvfp4(A, 16, 128, B, C, C + 124, E, None) == q4.Q4_ERR_OVERLAP  # tscale in scales
    # gemv: codes A, scales B (128 B), tscale C, x D (256 B), y E (64 B)
    assert L.q4_gemv_nvfp4(A, B, C, 16, 100, D, E, None) == q4.Q4_ERR_SHAPE
    assert L.q4_gemv_nvfp4(A, B, C, 0, 128, 0, 0, None) == q4.Q4_OK
    assert L.q4_gemv_nvfp4(A, B, 0, 16, 128, D, E, None) == q4.Q4_ERR_NULL
    assert L.q4_gemv_nvfp4(A, B + 1, C, 16, 128, D, E, None) == q4.Q4_ERR_ALIGN
    assert L.q4_gemv_nvfp4(A, B, C, 16, 128, D, B + 64, None) == q4.Q4_ERR_OVERLAP  # y over scales
    assert L.q4_gemv_nvfp4(A, B, C, 16, 128, D, C - 32, None) == q4.Q4_ERR_OVERLAP  # y over tscale
    # every call above fails a host check and launches nothing


def test_gemm_formats_errors(q4):
    L = q4.lib()
    E = 0x50000000
    M, K, N = 16, 128, 4  # codes 1 KB, scales/zeros 64 B, NVFP4 scales 128 B, X 1 KB, Y 256 B
    aff = lambda c, s, z, m, k, x, n, y: L.q4_gemm_smalln_affine(c, s, z, m, k, x, n, y, None)
    nv = lambda c, s, t, m, k, x, n, y: L.q4_gemm_smalln_nvfp4(c, s, t, m, k, x, n, y, None)
    for f in (aff, nv):
        assert f(A, B, C, M, K, D, 33, E) == q4.Q4_ERR_SHAPE
        assert f(A, B, C, M, K, D, -1, E) == q4.Q4_ERR_SHAPE
        assert f(A, B, C, M, 96, D, N, E) == q4.Q4_ERR_SHAPE
        assert f(None, None, None, M, K, None, 0, None) == q4.Q4_OK
        assert f(None, None, None, 0, K, None, N, None) == q4.Q4_OK
        assert f(None, B, C, M, K, D, N, E) == q4.Q4_ERR_NULL
        assert f(A, None, C, M, K, D, N, E) == q4.Q4_ERR_NULL
        assert f(A, B, None, M, K, D, N, E) == q4.Q4_ERR_NULL
        assert f(A, B, C, M, K, None, N, E) == q4.Q4_ERR_NULL
        assert f(A, B, C, M, K, D, N, None) == q4.Q4_ERR_NULL
        assert f(A + 8, B, C, M, K, D, N, E) == q4.Q4_ERR_ALIGN
        assert f(A, B + 1, C, M, K, D, N, E) == q4.Q4_ERR_ALIGN
        assert f(A, B, C, M, K, D + 8, N, E) == q4.Q4_ERR_ALIGN
        assert f(A, B, C, M, K, D, N, E + 2) == q4.Q4_ERR_ALIGN
        assert f(A, B, C, M, K, D, N, A + 1020) == q4.Q4_ERR_OVERLAP  # Y over the codes' tail
        assert f(A, B, C, M, K, D, N, D + 1020) == q4.Q4_ERR_OVERLAP  # Y over X's tail
    assert aff(A, B, C + 1, M, K, D, N, E) == q4.Q4_ERR_ALIGN
    assert aff(A, B, C, M, K, D, N, C + 60) == q4.Q4_ERR_OVERLAP      # Y over the zeros' tail
    assert nv(A, B, C + 2, M, K, D, N, E) == q4.Q4_ERR_ALIGN
    assert nv(A, B + 2, C, M, K, D, N, E) == q4.Q4_ERR_ALIGN          # NVFP4 scales: 4-byte aligned
    assert nv(A, B, C, M, K, D, N, B + 124) == q4.Q4_ERR_OVERLAP      # Y over the NVFP4 scales' tail
    assert nv(A, B, C, M, K, D, N, C) == q4.Q4_ERR_OVERLAP            # Y on the tensor scale


def test_x8_errors(q4):
    L = q4.lib()
    # x A (K=128: 256 B), q1 B (128 B), q2 C, d D (16 B)
    assert L.q4_quantize_x8(A, 100, 2, B, C, D, None) == q4.Q4_ERR_SHAPE
    assert L.q4_quantize_x8(A, 128, 3, B, C, D, None) == q4.Q4_ERR_SHAPE
    assert L.q4_quantize_x8(A, 128, 2, B, 0, D, None) == q4.Q4_ERR_NULL
    assert L.q4_quantize_x8(A, 128, 2, B + 8, C, D, None) == q4.Q4_ERR_ALIGN
    assert L.q4_quantize_x8(A, 128, 2, B, B + 64, D, None) == q4.Q4_ERR_OVERLAP
    assert L.q4_quantize_x8(A, 128, 1, B, 0, A + 128, None) == q4.Q4_ERR_OVERLAP   # d inside x
    # gemv: codes A, scales B, zeros C, q1 D, q2 E, d F, y G
    assert L.q4_gemv_affine_x8(A, B, C, 16, 100, D, E, F, G, None) == q4.Q4_ERR_SHAPE
    assert L.q4_gemv_affine_x8(A, B, C, 0, 128, 0, 0, 0, 0, None) == q4.Q4_OK
    assert L.q4_gemv_affine_x8(A, B, C, 16, 128, 0, E, F, G, None) == q4.Q4_ERR_NULL
    assert L.q4_gemv_affine_x8(A, B, C, 16, 128, D, E + 4, F, G, None) == q4.Q4_ERR_ALIGN
    assert L.q4_gemv_affine_x8(A, B, C, 16, 128, D, E, F, D + 64, None) == q4.Q4_ERR_OVERLAP  # y over q1
    # every call above fails a host check and launches nothing


def test_binding_refuses_without_library(tmp_path, monkeypatch):
    import bit_weight_gemv_amd as q4
    monkeypatch.setattr(q4, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(q4, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        q4.lib()
