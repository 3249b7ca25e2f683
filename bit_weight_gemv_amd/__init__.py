"""Python binding of libq4 (4-bit NF4-style codebook GEMV / small-N GEMM for
MI355X).  Argument marshalling only: every step runs in the HIP kernels of
libq4.so, reached through its C ABI (include/q4.h).  PyTorch supplies device
memory and the stream.

    codes, scales, status = q4_pack(W)            # W: fp32 [M, K] on the GPU
    y = q4_gemv(codes, scales, x)                 # x: bf16 [K]     -> fp32 [M]
    Y = q4_gemm_smalln(codes, scales, X)          # X: bf16 [N, K]  -> fp32 [N, M]

There is no fallback: if libq4.so is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libq4.so")

Q4_OK = 0
Q4_ERR_NULL = 1
Q4_ERR_SHAPE = 2
Q4_ERR_ALIGN = 3
Q4_ERR_OVERLAP = 4
Q4_ERR_DEVICE = 5
Q4_ERR_WORKSPACE = 6
Q4_MAX_K = 131072
Q4_MAX_N = 32
Q4_NOALLOC_SCRATCH_BYTES = 16 << 20
Q4_PACK_NONFINITE = 1
Q4_PACK_OVERFLOW = 2

EXPORTED = ("q4_codes_bytes", "q4_scales_bytes", "q4_codebook", "q4_status_string",
            "q4_pack", "q4_unpack_canonical", "q4_gemv", "q4_gemm_smalln", "q4_gemv_fused",
            "q4_gather_rows", "q4_pack_affine", "q4_gemv_affine", "q4_pack_nvfp4", "q4_gemv_nvfp4",
            "q4_quantize_x8", "q4_gemv_affine_x8", "q4_gemm_smalln_affine", "q4_gemm_smalln_nvfp4",
            "q4_gemv_fused_affine", "q4_gemv_fused_nvfp4", "q4_gemm_smalln_ws_bytes", "q4_gemm_smalln_ws",
            "q4_gemm_smalln_noalloc", "q4_gemm_smalln_affine_ws", "q4_gemm_smalln_nvfp4_ws")

Q4_OUT_F32 = 0
Q4_OUT_BF16 = 1
Q4_GATHER_BAD_ID = 1

Q4_MAX_FUSED = 4
Q4_MAX_FUSED_K = 16384
Q4_FUSE_SEPARATE = 0
Q4_FUSE_SWIGLU = 1


class Operand(ctypes.Structure):
    """q4_operand of include/q4.h."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("M", ctypes.c_int64),
                ("bias", ctypes.c_void_p)]


class OperandAffine(ctypes.Structure):
    """q4_operand_affine of include/q4.h."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("bias", ctypes.c_void_p)]


class OperandNvfp4(ctypes.Structure):
    """q4_operand_nvfp4 of include/q4.h."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("tscale", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("bias", ctypes.c_void_p)]

_lib = None
_lock = threading.Lock()


class Q4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """The loaded libq4.so with argument types set (raises if it is absent)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libq4.so not built ({LIB_PATH}); run python -m bit_weight_gemv_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.q4_codes_bytes.argtypes = [I64, I64]
        L.q4_codes_bytes.restype = ctypes.c_size_t
        L.q4_scales_bytes.argtypes = [I64, I64]
        L.q4_scales_bytes.restype = ctypes.c_size_t
        L.q4_codebook.argtypes = [P]
        L.q4_codebook.restype = None
        L.q4_status_string.argtypes = [I32]
        L.q4_status_string.restype = ctypes.c_char_p
        L.q4_pack.argtypes = [P, I64, I64, P, P, P, P]
        L.q4_pack.restype = I32
        L.q4_unpack_canonical.argtypes = [P, P, I64, I64, P, P, P]
        L.q4_unpack_canonical.restype = I32
        L.q4_gemv.argtypes = [P, P, I64, I64, P, P, P]
        L.q4_gemv.restype = I32
        L.q4_gemm_smalln.argtypes = [P, P, I64, I64, P, I64, P, P]
        L.q4_gemm_smalln.restype = I32
        L.q4_gemm_smalln_ws_bytes.argtypes = [I64, I64, I64]
        L.q4_gemm_smalln_ws_bytes.restype = ctypes.c_size_t
        L.q4_gemm_smalln_ws.argtypes = [P, P, I64, I64, P, I64, P, P, ctypes.c_size_t, P]
        L.q4_gemm_smalln_ws.restype = I32
        L.q4_gemm_smalln_noalloc.argtypes = [P, P, I64, I64, P, I64, P, P]
        L.q4_gemm_smalln_noalloc.restype = I32
        for name in ("q4_gemm_smalln_affine_ws", "q4_gemm_smalln_nvfp4_ws"):
            getattr(L, name).argtypes = [P, P, P, I64, I64, P, I64, P, P, ctypes.c_size_t, P]
            getattr(L, name).restype = I32
        for name in ("q4_gemv_fused", "q4_gemv_fused_affine", "q4_gemv_fused_nvfp4"):
            getattr(L, name).argtypes = [P, I32, I64, P, I32, P, P, P]
            getattr(L, name).restype = I32
        L.q4_gather_rows.argtypes = [P, P, I64, I64, P, I64, I32, P, P, P]
        L.q4_gather_rows.restype = I32
        L.q4_pack_affine.argtypes = [P, I64, I64, P, P, P, P, P]
        L.q4_pack_affine.restype = I32
        L.q4_gemv_affine.argtypes = [P, P, P, I64, I64, P, P, P]
        L.q4_gemv_affine.restype = I32
        L.q4_pack_nvfp4.argtypes = [P, I64, I64, P, P, P, P, P]
        L.q4_pack_nvfp4.restype = I32
        L.q4_gemv_nvfp4.argtypes = [P, P, P, I64, I64, P, P, P]
        L.q4_gemv_nvfp4.restype = I32
        L.q4_quantize_x8.argtypes = [P, I64, I32, P, P, P, P]
        L.q4_quantize_x8.restype = I32
        L.q4_gemv_affine_x8.argtypes = [P, P, P, I64, I64, P, P, P, P, P]
        L.q4_gemv_affine_x8.restype = I32
        L.q4_gemm_smalln_affine.argtypes = [P, P, P, I64, I64, P, I64, P, P]
        L.q4_gemm_smalln_affine.restype = I32
        L.q4_gemm_smalln_nvfp4.argtypes = [P, P, P, I64, I64, P, I64, P, P]
        L.q4_gemm_smalln_nvfp4.restype = I32
        _lib = L
        return L


def status_string(status: int) -> str:
    return lib().q4_status_string(int(status)).decode()


def codebook():
    """The 16 frozen levels (fp32) as a Python list."""
    out = (ctypes.c_float * 16)()
    lib().q4_codebook(out)
    return list(out)


def codes_bytes(M: int, K: int) -> int:
    return int(lib().q4_codes_bytes(M, K))


def scales_bytes(M: int, K: int) -> int:
    return int(lib().q4_scales_bytes(M, K))


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(t, name, dtype, device):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def q4_pack(W, codes=None, scales=None, status=None, stream=None):
    """Quantise fp32 W [M, K] -> (codes uint8 [M, K/2], scales fp16 [M, K/64],
    status int32 [1]).  status holds Q4_PACK_* flags once the stream reaches it."""
    torch = _torch()
    if W.dim() != 2:
        raise ValueError("W must be 2-D [M, K]")
    M, K = W.shape
    _check(W, "W", torch.float32, W.device)
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.empty((M, K // 64), dtype=torch.float16, device=W.device)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=W.device)
    _check(codes, "codes", torch.uint8, W.device)
    _check(scales, "scales", torch.float16, W.device)
    _check(status, "status", torch.int32, W.device)
    if codes.numel() * 2 != M * K or scales.numel() * 64 != M * K:
        raise ValueError("codes/scales do not match W's shape")
    st = lib().q4_pack(_ptr(W), M, K, _ptr(codes), _ptr(scales), _ptr(status), _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_pack")
    return codes, scales, status


def _mk(codes, scales):
    torch = _torch()
    if codes.dim() != 2 or scales.dim() != 2:
        raise ValueError("codes must be [M, K/2] and scales [M, K/64]")
    M, K = codes.shape[0], codes.shape[1] * 2
    if scales.shape[0] != M or scales.shape[1] * 64 != K:
        raise ValueError("codes and scales disagree on M, K")
    _check(codes, "codes", torch.uint8, codes.device)
    _check(scales, "scales", torch.float16, codes.device)
    return M, K


def q4_unpack_canonical(codes, scales, codes_out=None, scales_out=None, stream=None):
    """The canonical layout of a packed matrix: (codes uint8 [M, K/2],
    scales fp16 [M, K/64]) written into new (or the given) tensors."""
    torch = _torch()
    M, K = _mk(codes, scales)
    if codes_out is None:
        codes_out = torch.empty_like(codes)
    if scales_out is None:
        scales_out = torch.empty_like(scales)
    _check(codes_out, "codes_out", torch.uint8, codes.device)
    _check(scales_out, "scales_out", torch.float16, codes.device)
    if codes_out.numel() != codes.numel() or scales_out.numel() != scales.numel():
        raise ValueError("codes_out/scales_out do not match the packed matrix")
    st = lib().q4_unpack_canonical(_ptr(codes), _ptr(scales), M, K, _ptr(codes_out), _ptr(scales_out),
                                   _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_unpack_canonical")
    return codes_out, scales_out


def q4_gemv(codes, scales, x, y=None, stream=None):
    """y = dequant(W) . x for bf16 x [K]; returns fp32 y [M]."""
    torch = _torch()
    M, K = _mk(codes, scales)
    if x.numel() != K:
        raise ValueError(f"x must have K={K} entries")
    _check(x, "x", torch.bfloat16, codes.device)
    if y is None:
        y = torch.empty(M, dtype=torch.float32, device=codes.device)
    _check(y, "y", torch.float32, codes.device)
    if y.numel() != M:
        raise ValueError(f"y must have M={M} entries")
    st = lib().q4_gemv(_ptr(codes), _ptr(scales), M, K, _ptr(x), _ptr(y), _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_gemv")
    return y


def q4_gemm_smalln(codes, scales, X, Y=None, stream=None):
    """Y[n] = dequant(W) . X[n] for bf16 X [N, K], N <= 32; returns fp32 Y [N, M]."""
    torch = _torch()
    M, K = _mk(codes, scales)
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError(f"X must be [N, K={K}]")
    N = X.shape[0]
    _check(X, "X", torch.bfloat16, codes.device)
    if Y is None:
        Y = torch.empty((N, M), dtype=torch.float32, device=codes.device)
    _check(Y, "Y", torch.float32, codes.device)
    if Y.numel() != N * M:
        raise ValueError("Y must be [N, M]")
    st = lib().q4_gemm_smalln(_ptr(codes), _ptr(scales), M, K, _ptr(X), N, _ptr(Y), _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_gemm_smalln")
    return Y


def q4_gemm_smalln_ws_bytes(M: int, K: int, N: int) -> int:
    """Bytes of scratch q4_gemm_smalln_ws needs for this shape (0: none)."""
    return int(lib().q4_gemm_smalln_ws_bytes(M, K, N))


def gemm_workspace(M: int, K: int, N: int, device):
    """A uint8 device tensor of q4_gemm_smalln_ws_bytes(M, K, N) bytes, or None
    where the shape needs none."""
    n = q4_gemm_smalln_ws_bytes(M, K, N)
    if n == 0:
        return None
    return _torch().empty(n, dtype=_torch().uint8, device=device)


def q4_gemm_smalln_ws(codes, scales, X, workspace, Y=None, stream=None):
    """q4_gemm_smalln with scratch memory (a uint8 device tensor, or None where
    q4_gemm_smalln_ws_bytes is 0); returns fp32 Y [N, M]."""
    torch = _torch()
    M, K = _mk(codes, scales)
    N, Y = _smalln_out(X, K, M, Y, codes.device)
    ws, nb = None, 0
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, codes.device)
        ws, nb = _ptr(workspace), workspace.numel()
    st = lib().q4_gemm_smalln_ws(_ptr(codes), _ptr(scales), M, K, _ptr(X), N, _ptr(Y), ws, nb, _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_gemm_smalln_ws")
    return Y


def _ws_args(workspace, device):
    if workspace is None:
        return None, 0
    _check(workspace, "workspace", _torch().uint8, device)
    return _ptr(workspace), workspace.numel()


def q4_gemm_smalln_affine_ws(codes, scales, zeros, X, workspace, Y=None, stream=None):
    """q4_gemm_smalln_affine with scratch for the long-row K split."""
    torch = _torch()
    M, K = _mk(codes, scales)
    _check(zeros, "zeros", torch.float16, codes.device)
    if tuple(zeros.shape) != tuple(scales.shape):
        raise ValueError("zeros must have the shape of scales")
    N, Y = _smalln_out(X, K, M, Y, codes.device)
    ws, nb = _ws_args(workspace, codes.device)
    st = lib().q4_gemm_smalln_affine_ws(_ptr(codes), _ptr(scales), _ptr(zeros), M, K, _ptr(X), N, _ptr(Y), ws, nb,
                                        _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_gemm_smalln_affine_ws")
    return Y


def q4_gemm_smalln_noalloc(codes, scales, X, Y=None, stream=None):
    """q4_gemm_smalln_ws with the library's fixed device scratch
    (Q4_NOALLOC_SCRATCH_BYTES per device; calls on one device must not
    overlap in time); returns fp32 Y [N, M]."""
    M, K = _mk(codes, scales)
    N, Y = _smalln_out(X, K, M, Y, codes.device)
    st = lib().q4_gemm_smalln_noalloc(_ptr(codes), _ptr(scales), M, K, _ptr(X), N, _ptr(Y), _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_gemm_smalln_noalloc")
    return Y


def _fused(fmt, ops, x, mode, ys, residuals, stream):
    """The fused launch of one weight format (see q4_gemv_fused)."""
    torch = _torch()
    if mode not in ("separate", "swiglu"):
        raise ValueError("mode must be 'separate' or 'swiglu'")
    n = len(ops)
    struct = {"nf4": Operand, "affine": OperandAffine, "nvfp4": OperandNvfp4}[fmt]
    arr = (struct * max(n, 1))()
    K = None
    for i, op in enumerate(ops):
        codes, scales, extra, bias = (op[0], op[1], None, op[2]) if fmt == "nf4" else op
        if fmt == "nvfp4":
            if codes.dim() != 2 or scales.dim() != 2:
                raise ValueError("codes must be [M, K/2] and scales [M, K/16]")
            M, Ki = codes.shape[0], codes.shape[1] * 2
            if scales.shape[0] != M or scales.shape[1] * 16 != Ki:
                raise ValueError("codes and scales disagree on M, K")
            _check(codes, "codes", torch.uint8, codes.device)
            _check(scales, "scales", torch.uint8, codes.device)
            _check(extra, f"tscale[{i}]", torch.float32, codes.device)
        else:
            M, Ki = _mk(codes, scales)
            if fmt == "affine":
                _check(extra, f"zeros[{i}]", torch.float16, codes.device)
                if tuple(extra.shape) != tuple(scales.shape):
                    raise ValueError(f"zeros[{i}] must have the shape of scales")
        if K is not None and Ki != K:
            raise ValueError("all matrices must have the same K")
        K = Ki
        if bias is not None:
            _check(bias, f"bias[{i}]", torch.float32, codes.device)
            if bias.numel() != M:
                raise ValueError(f"bias[{i}] must have M={M} entries")
        bp = bias.data_ptr() if bias is not None else 0
        if fmt == "nf4":
            arr[i] = Operand(codes.data_ptr(), scales.data_ptr(), M, bp)
        else:
            arr[i] = struct(codes.data_ptr(), scales.data_ptr(), extra.data_ptr(), M, bp)
    dev = ops[0][0].device
    _check(x, "x", torch.bfloat16, dev)
    if x.numel() != K:
        raise ValueError(f"x must have K={K} entries")
    nout = 1 if mode == "swiglu" else n
    if ys is None:
        ys = [torch.empty(ops[i][0].shape[0], dtype=torch.float32, device=dev) for i in range(nout)]
    if len(ys) != nout or (residuals is not None and len(residuals) != nout):
        raise ValueError(f"mode {mode!r} with {n} matrices has {nout} outputs")
    for i, yv in enumerate(ys):
        _check(yv, f"y[{i}]", torch.float32, dev)
        if yv.numel() != ops[i][0].shape[0]:
            raise ValueError(f"y[{i}] must have M={ops[i][0].shape[0]} entries")
    yp = (ctypes.c_void_p * nout)(*[yv.data_ptr() for yv in ys])
    rp = None
    if residuals is not None:
        rp = (ctypes.c_void_p * nout)(*[(r.data_ptr() if r is not None else 0) for r in residuals])
        for i, r in enumerate(residuals):
            if r is not None:
                _check(r, f"residual[{i}]", torch.float32, dev)
                if r.numel() != ys[i].numel():
                    raise ValueError(f"residual[{i}] must have as many entries as y[{i}]")
    name = {"nf4": "q4_gemv_fused", "affine": "q4_gemv_fused_affine", "nvfp4": "q4_gemv_fused_nvfp4"}[fmt]
    st = getattr(lib(), name)(ctypes.cast(arr, ctypes.c_void_p), n, K, _ptr(x),
                              Q4_FUSE_SWIGLU if mode == "swiglu" else Q4_FUSE_SEPARATE,
                              ctypes.cast(yp, ctypes.c_void_p),
                              ctypes.cast(rp, ctypes.c_void_p) if rp is not None else None, _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, name)
    return ys


def q4_gemv_fused(ops, x, mode="separate", ys=None, residuals=None, stream=None):
    """Several products of one bf16 x [K] in one launch.  ops: list of
    (codes, scales, bias or None).  mode "separate": returns [y_i] with
    y_i = W_i . x + bias_i (+ residuals[i]); mode "swiglu" (two ops, gate then
    up): returns [y] with y = silu(W_0 . x + b_0) * (W_1 . x + b_1)
    (+ residuals[0]).  residuals: None or a list of fp32 tensors / None; an
    entry may be the output tensor itself (in-place add)."""
    return _fused("nf4", ops, x, mode, ys, residuals, stream)


def q4_gemv_fused_affine(ops, x, mode="separate", ys=None, residuals=None, stream=None):
    """q4_gemv_fused for affine-format matrices: ops is a list of (codes,
    scales, zeros, bias or None)."""
    return _fused("affine", ops, x, mode, ys, residuals, stream)


def q4_gemv_fused_nvfp4(ops, x, mode="separate", ys=None, residuals=None, stream=None):
    """q4_gemv_fused for NVFP4-style matrices: ops is a list of (codes,
    E4M3 scales uint8 [M, K/16], tensor scale fp32 [1], bias or None); in the
    swiglu mode each matrix keeps its own tensor scale."""
    return _fused("nvfp4", ops, x, mode, ys, residuals, stream)


def q4_gather_rows(codes, scales, ids, out_dtype=None, out=None, status=None, stream=None):
    """Rows ids (int32 [n]) of a packed matrix, dequantised: returns (out
    [n, K] fp32 or bf16, status int32 [1]).  status is 0, or Q4_GATHER_BAD_ID
    when some id is outside [0, M); the rows of such ids are zeros."""
    torch = _torch()
    M, K = _mk(codes, scales)
    dev = codes.device
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    _check(ids, "ids", torch.int32, dev)
    n = ids.numel()
    if out is None:
        out = torch.empty((n, K), dtype=out_dtype, device=dev)
    _check(out, "out", out_dtype, dev)
    if out.numel() != n * K:
        raise ValueError(f"out must hold n*K = {n * K} values")
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=dev)
    _check(status, "status", torch.int32, dev)
    st = lib().q4_gather_rows(_ptr(codes), _ptr(scales), M, K, _ptr(ids) if n else None, n,
                              Q4_OUT_BF16 if out_dtype == torch.bfloat16 else Q4_OUT_F32,
                              _ptr(out) if n else None, _ptr(status), _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_gather_rows")
    return out, status


def q4_pack_affine(W, codes=None, scales=None, zeros=None, status=None, stream=None):
    """Quantise fp32 W [M, K] into the affine format -> (codes uint8 [M, K/2],
    scales fp16 [M, K/64], zeros fp16 [M, K/64], status int32 [1])."""
    torch = _torch()
    if W.dim() != 2:
        raise ValueError("W must be [M, K]")
    M, K = W.shape
    dev = W.device
    _check(W, "W", torch.float32, dev)
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M, K // 64), dtype=torch.float16, device=dev)
    if zeros is None:
        zeros = torch.empty((M, K // 64), dtype=torch.float16, device=dev)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=dev)
    _check(codes, "codes", torch.uint8, dev)
    _check(scales, "scales", torch.float16, dev)
    _check(zeros, "zeros", torch.float16, dev)
    _check(status, "status", torch.int32, dev)
    if codes.numel() * 2 != M * K or scales.numel() * 64 != M * K or zeros.numel() * 64 != M * K:
        raise ValueError("codes / scales / zeros sizes do not match W")
    st = lib().q4_pack_affine(_ptr(W), M, K, _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(status), _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_pack_affine")
    return codes, scales, zeros, status


def q4_gemv_affine(codes, scales, zeros, x, y=None, stream=None):
    """y fp32 [M] = W . x for an affine-format W and bf16 x [K]."""
    torch = _torch()
    M, K = _mk(codes, scales)
    _check(zeros, "zeros", torch.float16, codes.device)
    if tuple(zeros.shape) != tuple(scales.shape):
        raise ValueError("zeros must have the shape of scales")
    _check(x, "x", torch.bfloat16, codes.device)
    if x.numel() != K:
        raise ValueError(f"x must have K={K} entries")
    if y is None:
        y = torch.empty(M, dtype=torch.float32, device=codes.device)
    _check(y, "y", torch.float32, codes.device)
    if y.numel() != M:
        raise ValueError(f"y must have M={M} entries")
    st = lib().q4_gemv_affine(_ptr(codes), _ptr(scales), _ptr(zeros), M, K, _ptr(x), _ptr(y), _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_gemv_affine")
    return y


def q4_pack_nvfp4(W, codes=None, scales=None, tscale=None, status=None, stream=None):
    """Quantise fp32 W [M, K] into the NVFP4-style format -> (codes uint8
    [M, K/2], scales E4M3 bytes uint8 [M, K/16], tensor scale fp32 [1],
    status int32 [1])."""
    torch = _torch()
    if W.dim() != 2:
        raise ValueError("W must be [M, K]")
    M, K = W.shape
    dev = W.device
    _check(W, "W", torch.float32, dev)
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    if tscale is None:
        tscale = torch.empty(1, dtype=torch.float32, device=dev)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=dev)
    for t, n, dt in ((codes, "codes", torch.uint8), (scales, "scales", torch.uint8),
                     (tscale, "tscale", torch.float32), (status, "status", torch.int32)):
        _check(t, n, dt, dev)
    if codes.numel() * 2 != M * K or scales.numel() * 16 != M * K:
        raise ValueError("codes / scales sizes do not match W")
    st = lib().q4_pack_nvfp4(_ptr(W), M, K, _ptr(codes), _ptr(scales), _ptr(tscale), _ptr(status), _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_pack_nvfp4")
    return codes, scales, tscale, status


def q4_gemv_nvfp4(codes, scales, tscale, x, y=None, stream=None):
    """y fp32 [M] = W . x for an NVFP4-style W (codes [M, K/2], scales uint8
    [M, K/16], tensor scale fp32 [1]) and bf16 x [K]."""
    torch = _torch()
    dev = codes.device
    if codes.dim() != 2 or scales.dim() != 2:
        raise ValueError("codes must be [M, K/2] and scales [M, K/16]")
    M, K = codes.shape[0], codes.shape[1] * 2
    if scales.shape[0] != M or scales.shape[1] * 16 != K:
        raise ValueError("codes and scales disagree on M, K")
    _check(codes, "codes", torch.uint8, dev)
    _check(scales, "scales", torch.uint8, dev)
    _check(tscale, "tscale", torch.float32, dev)
    _check(x, "x", torch.bfloat16, dev)
    if x.numel() != K:
        raise ValueError(f"x must have K={K} entries")
    if y is None:
        y = torch.empty(M, dtype=torch.float32, device=dev)
    _check(y, "y", torch.float32, dev)
    if y.numel() != M:
        raise ValueError(f"y must have M={M} entries")
    st = lib().q4_gemv_nvfp4(_ptr(codes), _ptr(scales), _ptr(tscale), M, K, _ptr(x), _ptr(y), _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_gemv_nvfp4")
    return y


def _smalln_out(X, K, M, Y, dev):
    torch = _torch()
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError(f"X must be [N, K={K}]")
    N = X.shape[0]
    _check(X, "X", torch.bfloat16, dev)
    if Y is None:
        Y = torch.empty((N, M), dtype=torch.float32, device=dev)
    _check(Y, "Y", torch.float32, dev)
    if Y.numel() != N * M:
        raise ValueError("Y must be [N, M]")
    return N, Y


def q4_gemm_smalln_affine(codes, scales, zeros, X, Y=None, stream=None):
    """Y[n] = W . X[n] for an affine-format W and bf16 X [N, K], N <= 32;
    returns fp32 Y [N, M]."""
    torch = _torch()
    M, K = _mk(codes, scales)
    _check(zeros, "zeros", torch.float16, codes.device)
    if tuple(zeros.shape) != tuple(scales.shape):
        raise ValueError("zeros must have the shape of scales")
    N, Y = _smalln_out(X, K, M, Y, codes.device)
    st = lib().q4_gemm_smalln_affine(_ptr(codes), _ptr(scales), _ptr(zeros), M, K, _ptr(X), N, _ptr(Y),
                                     _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_gemm_smalln_affine")
    return Y


def q4_gemm_smalln_nvfp4(codes, scales, tscale, X, Y=None, stream=None):
    """Y[n] = W . X[n] for an NVFP4-style W (codes [M, K/2], scales uint8
    [M, K/16], tensor scale fp32 [1]) and bf16 X [N, K], N <= 32."""
    torch = _torch()
    dev = codes.device
    if codes.dim() != 2 or scales.dim() != 2:
        raise ValueError("codes must be [M, K/2] and scales [M, K/16]")
    M, K = codes.shape[0], codes.shape[1] * 2
    if scales.shape[0] != M or scales.shape[1] * 16 != K:
        raise ValueError("codes and scales disagree on M, K")
    _check(codes, "codes", torch.uint8, dev)
    _check(scales, "scales", torch.uint8, dev)
    _check(tscale, "tscale", torch.float32, dev)
    N, Y = _smalln_out(X, K, M, Y, dev)
    st = lib().q4_gemm_smalln_nvfp4(_ptr(codes), _ptr(scales), _ptr(tscale), M, K, _ptr(X), N, _ptr(Y),
                                    _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_gemm_smalln_nvfp4")
    return Y


def q4_gemm_smalln_nvfp4_ws(codes, scales, tscale, X, workspace, Y=None, stream=None):
    """q4_gemm_smalln_nvfp4 with scratch for the long-row K split."""
    torch = _torch()
    dev = codes.device
    if codes.dim() != 2 or scales.dim() != 2:
        raise ValueError("codes must be [M, K/2] and scales [M, K/16]")
    M, K = codes.shape[0], codes.shape[1] * 2
    if scales.shape[0] != M or scales.shape[1] * 16 != K:
        raise ValueError("codes and scales disagree on M, K")
    _check(codes, "codes", torch.uint8, dev)
    _check(scales, "scales", torch.uint8, dev)
    _check(tscale, "tscale", torch.float32, dev)
    N, Y = _smalln_out(X, K, M, Y, dev)
    ws, nb = _ws_args(workspace, dev)
    st = lib().q4_gemm_smalln_nvfp4_ws(_ptr(codes), _ptr(scales), _ptr(tscale), M, K, _ptr(X), N, _ptr(Y), ws, nb,
                                       _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_gemm_smalln_nvfp4_ws")
    return Y


def q4_quantize_x8(x, words=2, q1=None, q2=None, d=None, stream=None):
    """bf16 x [K] -> (q1 int8 [K], q2 int8 [K] or None, d fp32 [K/32])."""
    torch = _torch()
    dev = x.device
    _check(x, "x", torch.bfloat16, dev)
    K = x.numel()
    if words not in (1, 2):
        raise ValueError("words must be 1 or 2")
    if q1 is None:
        q1 = torch.empty(K, dtype=torch.int8, device=dev)
    if q2 is None and words == 2:
        q2 = torch.empty(K, dtype=torch.int8, device=dev)
    if d is None:
        d = torch.empty(K // 32, dtype=torch.float32, device=dev)
    _check(q1, "q1", torch.int8, dev)
    _check(d, "d", torch.float32, dev)
    if words == 2:
        _check(q2, "q2", torch.int8, dev)
    st = lib().q4_quantize_x8(_ptr(x), K, words, _ptr(q1), _ptr(q2) if words == 2 else None, _ptr(d),
                              _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_quantize_x8")
    return q1, (q2 if words == 2 else None), d


def q4_gemv_affine_x8(codes, scales, zeros, q1, q2, d, y=None, stream=None):
    """y fp32 [M] = W . xq for an affine-format W and int8 activations from
    q4_quantize_x8 (q2 None: one word)."""
    torch = _torch()
    M, K = _mk(codes, scales)
    dev = codes.device
    _check(zeros, "zeros", torch.float16, dev)
    _check(q1, "q1", torch.int8, dev)
    _check(d, "d", torch.float32, dev)
    if q2 is not None:
        _check(q2, "q2", torch.int8, dev)
    if q1.numel() != K or d.numel() != K // 32 or (q2 is not None and q2.numel() != K):
        raise ValueError("activation words do not match K")
    if y is None:
        y = torch.empty(M, dtype=torch.float32, device=dev)
    _check(y, "y", torch.float32, dev)
    st = lib().q4_gemv_affine_x8(_ptr(codes), _ptr(scales), _ptr(zeros), M, K, _ptr(q1),
                                 _ptr(q2) if q2 is not None else None, _ptr(d), _ptr(y), _stream(stream))
    if st != Q4_OK:
        raise Q4Error(st, "q4_gemv_affine_x8")
    return y
