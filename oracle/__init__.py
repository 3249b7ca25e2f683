"""fp64 CPU oracle for the 4-bit NF4-style codebook GEMV / small-N GEMM.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg load it; the product path never does.  The arithmetic lives
in ``oracle.c`` (plain C, fp64); this module compiles it with gcc and wraps
it with numpy arrays via ctypes.  It imports nothing from the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at another build of oracle.c (the mutation
# test builds deliberately broken copies to show the pins catch them).
_OVERRIDE = os.environ.get("Q4_ORACLE_LIB")
_lib = None
_lock = threading.Lock()

PACK_NONFINITE = 1
PACK_OVERFLOW = 2


def compile_source(src: str, out: str) -> str:
    """gcc one oracle source file into a shared library (strict IEEE)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", "-I", _HERE, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if _OVERRIDE:
            lib = ctypes.CDLL(_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_codebook_f64.argtypes = [P]
        lib.oracle_codebook_f32.argtypes = [P]
        lib.oracle_phi_inv.argtypes = [ctypes.c_double]
        lib.oracle_phi_inv.restype = ctypes.c_double
        lib.oracle_f32_to_f16_rne.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16_rne.restype = ctypes.c_uint16
        lib.oracle_f32_to_f16_rne_array.argtypes = [P, I64, P]
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_pack_rows.argtypes = [P, I64, I64, I64, I64, P, P]
        lib.oracle_pack_rows.restype = ctypes.c_int
        lib.oracle_dequant.argtypes = [P, P, I64, I64, P]
        lib.oracle_gemv_rows.argtypes = [P, P, I64, I64, P, I64, I64, P, P]
        lib.oracle_gemm.argtypes = [P, P, I64, I64, P, I64, P, P]
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_epilogue.argtypes = [P, P, P, P, P, I64, ctypes.c_int, P]
        lib.oracle_epilogue.restype = None
        lib.oracle_argmax_f64.argtypes = [P, I64]
        lib.oracle_argmax_f64.restype = I64
        lib.oracle_argmax_f32.argtypes = [P, I64]
        lib.oracle_argmax_f32.restype = I64
        lib.oracle_f64_to_f16_rne.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_f16_rne.restype = ctypes.c_uint16
        lib.oracle_pack_affine_rows.argtypes = [P, I64, I64, I64, I64, P, P, P]
        lib.oracle_pack_affine_rows.restype = ctypes.c_int
        lib.oracle_dequant_affine.argtypes = [P, P, P, I64, I64, P]
        lib.oracle_dequant_affine.restype = None
        lib.oracle_gemv_affine_rows.argtypes = [P, P, P, I64, I64, P, I64, I64, P, P]
        lib.oracle_gemv_affine_rows.restype = None
        lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_to_f64.restype = ctypes.c_double
        lib.oracle_e2m1_to_f64.argtypes = [ctypes.c_uint8]
        lib.oracle_e2m1_to_f64.restype = ctypes.c_double
        lib.oracle_nvfp4_tensor_scale.argtypes = [P, I64, P]
        lib.oracle_nvfp4_tensor_scale.restype = ctypes.c_float
        lib.oracle_pack_nvfp4_rows.argtypes = [P, I64, I64, I64, I64, ctypes.c_float, P, P]
        lib.oracle_pack_nvfp4_rows.restype = ctypes.c_int
        lib.oracle_dequant_nvfp4.argtypes = [P, P, ctypes.c_float, I64, I64, P]
        lib.oracle_dequant_nvfp4.restype = None
        lib.oracle_gemv_nvfp4_rows.argtypes = [P, P, ctypes.c_float, I64, I64, P, I64, I64, P, P]
        lib.oracle_gemv_nvfp4_rows.restype = None
        lib.oracle_quantize_x8.argtypes = [P, I64, ctypes.c_int, P, P, P]
        lib.oracle_quantize_x8.restype = None
        lib.oracle_dequantize_x8.argtypes = [P, P, P, I64, P]
        lib.oracle_dequantize_x8.restype = None
        lib.oracle_gemv_affine_x8_rows.argtypes = [P, P, P, I64, I64, P, P, P, I64, I64, P, P]
        lib.oracle_gemv_affine_x8_rows.restype = None
        lib.oracle_f64_to_bf16_rne.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_gather_rows.argtypes = [P, P, I64, I64, P, I64, ctypes.c_int, P]
        lib.oracle_gather_rows.restype = ctypes.c_int32
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check_shape(M: int, K: int):
    if M < 0 or K < 0 or K % 64 != 0:
        raise ValueError(f"oracle: need M >= 0 and K a multiple of 64, got M={M} K={K}")


def codebook_f64() -> np.ndarray:
    out = np.zeros(16, np.float64)
    _load().oracle_codebook_f64(_ptr(out))
    return out


def codebook_f32() -> np.ndarray:
    out = np.zeros(16, np.float32)
    _load().oracle_codebook_f32(_ptr(out))
    return out


def phi_inv(p: float) -> float:
    return _load().oracle_phi_inv(p)


def f32_to_f16_bits(v) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(v, np.float32).ravel())
    out = np.zeros(v.size, np.uint16)
    _load().oracle_f32_to_f16_rne_array(_ptr(v), v.size, _ptr(out))
    return out


def f16_bits_to_f64(h) -> np.ndarray:
    lib = _load()
    h = np.asarray(h, np.uint16).ravel()
    return np.array([lib.oracle_f16_to_f64(int(t)) for t in h], np.float64)


def bf16_bits_to_f64(b) -> np.ndarray:
    lib = _load()
    b = np.asarray(b, np.uint16).ravel()
    return np.array([lib.oracle_bf16_to_f64(int(t)) for t in b], np.float64)


def pack(W: np.ndarray, threads: int = 1):
    """W fp32 [M,K] -> (codes uint8 [M,K/2], scales fp16 bits uint16 [M,K/64], status)."""
    W = np.ascontiguousarray(W, np.float32)
    M, K = W.shape
    _check_shape(M, K)
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 64), np.uint16)
    lib = _load()
    status = [0]

    def run(r0, r1, slot):
        slot.append(lib.oracle_pack_rows(_ptr(W), M, K, r0, r1, _ptr(codes), _ptr(scales)))

    _run_rows(M, threads, run, status)
    st = 0
    for s in status[1:]:
        st |= s
    return codes, scales, st


def dequant(codes: np.ndarray, scales: np.ndarray, M: int, K: int) -> np.ndarray:
    _check_shape(M, K)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    out = np.zeros((M, K), np.float64)
    _load().oracle_dequant(_ptr(codes), _ptr(scales), M, K, _ptr(out))
    return out


def gemv(codes, scales, M: int, K: int, x_bits, rows=None, threads: int = 1):
    """y, S (fp64, length M).  rows=(r0, r1) restricts the work to those rows
    (other entries stay NaN)."""
    _check_shape(M, K)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    if x_bits.size != K:
        raise ValueError("oracle.gemv: x must have K entries")
    y = np.full(M, np.nan)
    S = np.full(M, np.nan)
    lib = _load()
    r0, r1 = (0, M) if rows is None else rows

    def run(a, b, slot):
        lib.oracle_gemv_rows(_ptr(codes), _ptr(scales), M, K, _ptr(x_bits), a, b, _ptr(y), _ptr(S))

    _run_rows(r1 - r0, threads, lambda a, b, s: run(r0 + a, r0 + b, s), [0])
    return y, S


def gemv_row_list(codes, scales, M: int, K: int, x_bits, rows):
    """y, S for an explicit list of rows (returned in that order)."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    lib = _load()
    y = np.full(M, np.nan)
    S = np.full(M, np.nan)
    rows = np.asarray(rows, np.int64)
    for r in rows:
        lib.oracle_gemv_rows(_ptr(codes), _ptr(scales), M, K, _ptr(x_bits), int(r), int(r) + 1,
                             _ptr(y), _ptr(S))
    return y[rows], S[rows]


def gemm(codes, scales, M: int, K: int, X_bits):
    """Y, S fp64 [N, M] for X bf16 bits [N, K]."""
    _check_shape(M, K)
    X_bits = np.ascontiguousarray(X_bits, np.uint16)
    N = X_bits.shape[0]
    if X_bits.shape[1] != K:
        raise ValueError("oracle.gemm: X must be [N, K]")
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    Y = np.zeros((N, M), np.float64)
    S = np.zeros((N, M), np.float64)
    _load().oracle_gemm(_ptr(codes), _ptr(scales), M, K, _ptr(X_bits), N, _ptr(Y), _ptr(S))
    return Y, S


def silu(z: float) -> float:
    """SiLU(z) = z / (1 + e^-z) in fp64."""
    return float(_load().oracle_silu(float(z)))


def epilogue(t0, t1=None, bias0=None, bias1=None, residual=None, swiglu: bool = False):
    """The fused-projection epilogue in fp64 (see oracle_epilogue): t0, t1
    fp64 products; bias0, bias1, residual fp32 or None."""
    t0 = np.ascontiguousarray(t0, np.float64)
    n = t0.size
    if swiglu:
        if t1 is None:
            raise ValueError("oracle.epilogue: swiglu needs t1")
        t1 = np.ascontiguousarray(t1, np.float64)
        if t1.size != n:
            raise ValueError("oracle.epilogue: t0 and t1 differ in length")

    def f32(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a, np.float32)
        if a.size != n:
            raise ValueError("oracle.epilogue: bias/residual length differs from t0")
        return a
    b0, b1, r = f32(bias0), f32(bias1), f32(residual)
    out = np.empty(n, np.float64)
    nullp = ctypes.c_void_p(0)
    _load().oracle_epilogue(_ptr(t0), _ptr(t1) if swiglu else nullp, _ptr(b0) if b0 is not None else nullp,
                            _ptr(b1) if b1 is not None else nullp, _ptr(r) if r is not None else nullp,
                            n, 1 if swiglu else 0, _ptr(out))
    return out


def f64_to_f16_bits(v: float) -> int:
    """One rounding of a double to IEEE binary16 bits, nearest-even."""
    return int(_load().oracle_f64_to_f16_rne(float(v)))


def pack_affine(W: np.ndarray, threads: int = 1):
    """(codes uint8 [M, K/2], scales fp16 bits [M, K/64], zeros fp16 bits
    [M, K/64], status) of the affine 4-bit format."""
    W = np.ascontiguousarray(W, np.float32)
    M, K = W.shape
    _check_shape(M, K)
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 64), np.uint16)
    zeros = np.zeros((M, K // 64), np.uint16)
    lib = _load()
    status = [0]

    def run(r0, r1, slot):
        slot.append(lib.oracle_pack_affine_rows(_ptr(W), M, K, r0, r1, _ptr(codes), _ptr(scales), _ptr(zeros)))

    _run_rows(M, threads, run, status)
    st = 0
    for v in status[1:]:
        st |= v
    return codes, scales, zeros, st


def dequant_affine(codes, scales, zeros, M: int, K: int) -> np.ndarray:
    _check_shape(M, K)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    zeros = np.ascontiguousarray(zeros, np.uint16)
    out = np.zeros((M, K), np.float64)
    _load().oracle_dequant_affine(_ptr(codes), _ptr(scales), _ptr(zeros), M, K, _ptr(out))
    return out


def gemv_affine(codes, scales, zeros, M: int, K: int, x_bits, rows=None, threads: int = 1):
    """y, S (fp64, length M) of the affine format; rows=(r0, r1) restricts
    the work (other entries NaN)."""
    _check_shape(M, K)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    zeros = np.ascontiguousarray(zeros, np.uint16)
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    if x_bits.size != K:
        raise ValueError("oracle.gemv_affine: x must have K entries")
    y = np.full(M, np.nan)
    S = np.full(M, np.nan)
    lib = _load()
    r0, r1 = (0, M) if rows is None else rows

    def run(a, b, slot):
        lib.oracle_gemv_affine_rows(_ptr(codes), _ptr(scales), _ptr(zeros), M, K, _ptr(x_bits), r0 + a, r0 + b,
                                    _ptr(y), _ptr(S))

    _run_rows(r1 - r0, threads, run, [0])
    return y, S


def gemm_affine(codes, scales, zeros, M: int, K: int, X_bits, threads: int = 1):
    """Y, S fp64 [N, M] of the affine format for X bf16 bits [N, K]: the
    prefill product is, by definition, one GEMV per token (accel/tensor
    func Int4MatMul: Y[n] = W . X[n])."""
    X_bits = np.ascontiguousarray(X_bits, np.uint16)
    if X_bits.ndim != 2 or X_bits.shape[1] != K:
        raise ValueError("oracle.gemm_affine: X must be [N, K]")
    N = X_bits.shape[0]
    Y = np.zeros((N, M), np.float64)
    S = np.zeros((N, M), np.float64)
    for n in range(N):
        Y[n], S[n] = gemv_affine(codes, scales, zeros, M, K, X_bits[n], threads=threads)
    return Y, S


def e4m3_to_f64(b: int) -> float:
    return float(_load().oracle_e4m3_to_f64(int(b)))


def e2m1_to_f64(c: int) -> float:
    return float(_load().oracle_e2m1_to_f64(int(c)))


def pack_nvfp4(W: np.ndarray, threads: int = 1):
    """(codes uint8 [M, K/2], scales E4M3 bytes uint8 [M, K/16], tensor scale
    (float), status) of the NVFP4-style format."""
    W = np.ascontiguousarray(W, np.float32)
    M, K = W.shape
    _check_shape(M, K)
    lib = _load()
    st0 = ctypes.c_int(0)
    s = float(lib.oracle_nvfp4_tensor_scale(_ptr(W), W.size, ctypes.byref(st0)))
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 16), np.uint8)
    status = [0]

    def run(r0, r1, slot):
        slot.append(lib.oracle_pack_nvfp4_rows(_ptr(W), M, K, r0, r1, s, _ptr(codes), _ptr(scales)))

    _run_rows(M, threads, run, status)
    st = st0.value
    for v in status[1:]:
        st |= v
    return codes, scales, s, st


def dequant_nvfp4(codes, scales, s: float, M: int, K: int) -> np.ndarray:
    _check_shape(M, K)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    out = np.zeros((M, K), np.float64)
    _load().oracle_dequant_nvfp4(_ptr(codes), _ptr(scales), float(s), M, K, _ptr(out))
    return out


def gemv_nvfp4(codes, scales, s: float, M: int, K: int, x_bits, rows=None, threads: int = 1):
    """y, S (fp64, length M) of the NVFP4-style format."""
    _check_shape(M, K)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    if x_bits.size != K:
        raise ValueError("oracle.gemv_nvfp4: x must have K entries")
    y = np.full(M, np.nan)
    S = np.full(M, np.nan)
    lib = _load()
    r0, r1 = (0, M) if rows is None else rows

    def run(a, b, slot):
        lib.oracle_gemv_nvfp4_rows(_ptr(codes), _ptr(scales), float(s), M, K, _ptr(x_bits), r0 + a, r0 + b,
                                   _ptr(y), _ptr(S))

    _run_rows(r1 - r0, threads, run, [0])
    return y, S


def gemm_nvfp4(codes, scales, s: float, M: int, K: int, X_bits, threads: int = 1):
    """Y, S fp64 [N, M] of the NVFP4-style format for X bf16 bits [N, K]:
    one GEMV per token, as gemm_affine."""
    X_bits = np.ascontiguousarray(X_bits, np.uint16)
    if X_bits.ndim != 2 or X_bits.shape[1] != K:
        raise ValueError("oracle.gemm_nvfp4: X must be [N, K]")
    N = X_bits.shape[0]
    Y = np.zeros((N, M), np.float64)
    S = np.zeros((N, M), np.float64)
    for n in range(N):
        Y[n], S[n] = gemv_nvfp4(codes, scales, s, M, K, X_bits[n], threads=threads)
    return Y, S


def quantize_x8(x_bits, words: int = 2):
    """(q1 int8 [K], q2 int8 [K] or None, d fp32 [K/32]) of bf16 x."""
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    K = x_bits.size
    if K % 32 != 0 or words not in (1, 2):
        raise ValueError("oracle.quantize_x8: K % 32 == 0 and words in (1, 2)")
    q1 = np.zeros(K, np.int8)
    q2 = np.zeros(K, np.int8) if words == 2 else None
    d = np.zeros(K // 32, np.float32)
    _load().oracle_quantize_x8(_ptr(x_bits), K, words, _ptr(q1), _ptr(q2) if q2 is not None else None, _ptr(d))
    return q1, q2, d


def dequantize_x8(q1, q2, d) -> np.ndarray:
    q1 = np.ascontiguousarray(q1, np.int8)
    d = np.ascontiguousarray(d, np.float32)
    out = np.zeros(q1.size, np.float64)
    q2c = np.ascontiguousarray(q2, np.int8) if q2 is not None else None
    _load().oracle_dequantize_x8(_ptr(q1), _ptr(q2c) if q2c is not None else None, _ptr(d), q1.size, _ptr(out))
    return out


def gemv_affine_x8(codes, scales, zeros, M: int, K: int, q1, q2, d, threads: int = 1):
    """y, S (fp64) of the affine format's GEMV on int8 activations."""
    _check_shape(M, K)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    zeros = np.ascontiguousarray(zeros, np.uint16)
    q1 = np.ascontiguousarray(q1, np.int8)
    q2c = np.ascontiguousarray(q2, np.int8) if q2 is not None else None
    d = np.ascontiguousarray(d, np.float32)
    y = np.full(M, np.nan)
    S = np.full(M, np.nan)
    lib = _load()

    def run(a, b, slot):
        lib.oracle_gemv_affine_x8_rows(_ptr(codes), _ptr(scales), _ptr(zeros), M, K, _ptr(q1),
                                       _ptr(q2c) if q2c is not None else None, _ptr(d), a, b, _ptr(y), _ptr(S))

    _run_rows(M, threads, run, [0])
    return y, S


GATHER_BAD_ID = 1


def f64_to_bf16_bits(v: float) -> int:
    """One rounding of a finite double to bfloat16 bits, nearest-even."""
    return int(_load().oracle_f64_to_bf16_rne(float(v)))


def gather_rows(codes, scales, M: int, K: int, ids, bf16: bool = False, out=None):
    """(out, flags): out[i] = What[ids[i]] rounded once to fp32 (or bf16 bits,
    uint16); rows of ids outside [0, M) are zeros and set GATHER_BAD_ID in
    flags."""
    _check_shape(M, K)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    ids = np.ascontiguousarray(ids, np.int32)
    n = ids.size
    if out is None:
        out = np.full((n, K), 0xFFFF, np.uint16) if bf16 else np.full((n, K), np.nan, np.float32)
    flags = _load().oracle_gather_rows(_ptr(codes), _ptr(scales), M, K, _ptr(ids), n, 1 if bf16 else 0,
                                       _ptr(out))
    return out, int(flags)


def argmax(y) -> int:
    y = np.ascontiguousarray(y)
    lib = _load()
    if y.dtype == np.float64:
        return int(lib.oracle_argmax_f64(_ptr(y), y.size))
    if y.dtype == np.float32:
        return int(lib.oracle_argmax_f32(_ptr(y), y.size))
    raise TypeError("oracle.argmax: float32 or float64 only")


def within_tolerance(y, y_ref, S, rel: float = 1e-3, abs_: float = 1e-5):
    """The acceptance bound |y - y_ref| <= rel * S + abs_, element-wise.
    Returns (ok, worst ratio of |y - y_ref| to the bound)."""
    y = np.asarray(y, np.float64)
    err = np.abs(y - y_ref)
    bound = rel * S + abs_
    ratio = err / bound
    ok = bool(np.all(np.isfinite(y)) and np.all(err <= bound))
    return ok, float(np.max(ratio)) if ratio.size else 0.0


def _run_rows(n: int, threads: int, fn, status):
    """Split [0, n) into `threads` contiguous ranges run on Python threads
    (ctypes releases the GIL while the C code runs)."""
    threads = max(1, min(int(threads), n if n > 0 else 1))
    if threads == 1:
        fn(0, n, status)
        return
    bounds = [n * t // threads for t in range(threads + 1)]
    ts = []
    slots = [[] for _ in range(threads)]
    for t in range(threads):
        th = threading.Thread(target=fn, args=(bounds[t], bounds[t + 1], slots[t]))
        th.start()
        ts.append(th)
    for th in ts:
        th.join()
    for s in slots:
        status.extend(s)
