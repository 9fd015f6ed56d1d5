"""Thin ctypes binding over libconvrot.so (the C ABI in include/convrot.h).

Argument marshalling only: every step of the quantized linear runs in the HIP kernels of the
library. PyTorch supplies device memory and the current HIP stream. There is no fallback: if
the library is missing or a call fails, a ConvRotError is raised.

Two layers:
  * ``rq_*`` -- the C entry points under their own names, taking integer device pointers;
  * ``quantize_weights``, ``rotq_linear``, ``rotate_quantize``, ``gemm_dequant``,
    ``gemm_s32`` -- tensor wrappers that allocate outputs with torch and pass the current
    stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(PKG, "libconvrot.so")

RQ_OK, RQ_EINVAL, RQ_EUNSUPPORTED, RQ_EWORKSPACE, RQ_EHIP = range(5)
RQ_F32, RQ_F16, RQ_BF16 = 0, 1, 2
RQ_ROT_WHT = 1
RQ_X_ROWS, RQ_X_TILED, RQ_X_FP6 = 0, 1, 2
RQ_W_ROWS, RQ_W_FP6 = 0, 1
RQ_W_ABSMAX, RQ_W_MSE, RQ_W_TENSOR = 0, 1, 2
RQ_ACT_NONE, RQ_ACT_GELU_ERF, RQ_ACT_GELU_TANH = 0, 1, 2


class ConvRotError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, _status_text(status), detail))


class rq_qconfig(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("rot_kind", ctypes.c_int32), ("rot_block", ctypes.c_int32),
                ("x_layout", ctypes.c_int32), ("w_scale_mode", ctypes.c_int32), ("w_layout", ctypes.c_int32),
                ("act", ctypes.c_int32)]


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libconvrot.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise FileNotFoundError(
            "libconvrot.so is not built (%s); run __graft_entry__.build() or "
            "python w4a4_integer_quantized_amd/build.py" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    CFG = ctypes.POINTER(rq_qconfig)
    sig = {
        "rq_quantize_weights": [P, I32, I64, I64, CFG, P, P, P],
        "rq_rotate_quantize": [P, I32, I64, I64, CFG, P, P, P],
        "rq_rotq_linear": [P, I32, I64, I64, P, P, I64, P, CFG, P, P, SZ, P],
        "rq_rotq_linear_noalloc": [P, I32, I64, I64, P, P, I64, P, CFG, P, P],
        "rq_gemm_dequant": [P, P, P, P, P, I64, I64, I64, CFG, P, I32, P],
        "rq_gemm_s32": [P, P, I64, I64, I64, CFG, P, P],
        "rq_check_rotq_linear_args": [P, I32, I64, I64, P, P, I64, P, CFG, P, P, SZ],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.rq_rotq_linear_workspace_size.argtypes = [I64, I64, CFG]
    lib.rq_rotq_linear_workspace_size.restype = SZ
    lib.rq_codes_bytes.argtypes = [I64, I64, CFG]
    lib.rq_codes_bytes.restype = SZ
    lib.rq_weight_bytes.argtypes = [I64, I64, CFG]
    lib.rq_weight_bytes.restype = SZ
    lib.rq_status_string.argtypes = [ctypes.c_int]
    lib.rq_status_string.restype = ctypes.c_char_p
    lib.rq_last_error_detail.argtypes = []
    lib.rq_last_error_detail.restype = ctypes.c_char_p
    lib.rq_version.argtypes = []
    lib.rq_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _status_text(s: int) -> str:
    try:
        return load().rq_status_string(s).decode()
    except Exception:  # pragma: no cover - only when the library itself is unusable
        return "status %d" % s


def _check(status: int, where: str):
    if status != RQ_OK:
        raise ConvRotError(status, where, load().rq_last_error_detail().decode())


def make_cfg(bits: int = 8, rot_block: int = 128, rot_kind: int = RQ_ROT_WHT,
             x_layout: int = RQ_X_ROWS, w_scale_mode: int = RQ_W_ABSMAX,
             w_layout: int = RQ_W_ROWS, act: int = RQ_ACT_NONE) -> rq_qconfig:
    return rq_qconfig(bits, rot_kind, rot_block, x_layout, w_scale_mode, w_layout, act)


# ----------------------------------------------------------------------------- raw entry points
def rq_quantize_weights(W, w_dtype, N, K, cfg, Wq, w_scale, stream) -> int:
    return load().rq_quantize_weights(W, w_dtype, N, K, ctypes.byref(cfg), Wq, w_scale, stream)


def rq_rotate_quantize(X, x_dtype, M, K, cfg, Xq, x_scale, stream) -> int:
    return load().rq_rotate_quantize(X, x_dtype, M, K, ctypes.byref(cfg), Xq, x_scale, stream)


def rq_rotq_linear(X, x_dtype, M, K, Wq, w_scale, N, bias, cfg, Y, ws, ws_bytes, stream) -> int:
    return load().rq_rotq_linear(X, x_dtype, M, K, Wq, w_scale, N, bias, ctypes.byref(cfg), Y, ws,
                                 ws_bytes, stream)


RQ_NOALLOC_SCRATCH_BYTES = 64 << 20     # the static scratch of rq_rotq_linear_noalloc (convrot.h)


def rq_rotq_linear_noalloc(X, x_dtype, M, K, Wq, w_scale, N, bias, cfg, Y, stream) -> int:
    return load().rq_rotq_linear_noalloc(X, x_dtype, M, K, Wq, w_scale, N, bias, ctypes.byref(cfg), Y, stream)


def rq_gemm_dequant(Xq, x_scale, Wq, w_scale, bias, M, N, K, cfg, Y, y_dtype, stream) -> int:
    return load().rq_gemm_dequant(Xq, x_scale, Wq, w_scale, bias, M, N, K, ctypes.byref(cfg), Y,
                                  y_dtype, stream)


def rq_gemm_s32(Xq, Wq, M, N, K, cfg, acc, stream) -> int:
    return load().rq_gemm_s32(Xq, Wq, M, N, K, ctypes.byref(cfg), acc, stream)


def rq_rotq_linear_workspace_size(M, K, cfg) -> int:
    return load().rq_rotq_linear_workspace_size(M, K, ctypes.byref(cfg))


def rq_codes_bytes(rows, K, cfg) -> int:
    return load().rq_codes_bytes(rows, K, ctypes.byref(cfg))


def rq_weight_bytes(N, K, cfg) -> int:
    return load().rq_weight_bytes(N, K, ctypes.byref(cfg))


def rq_check_rotq_linear_args(X, x_dtype, M, K, Wq, w_scale, N, bias, cfg, Y, ws, ws_bytes) -> int:
    return load().rq_check_rotq_linear_args(X, x_dtype, M, K, Wq, w_scale, N, bias,
                                            ctypes.byref(cfg), Y, ws, ws_bytes)


def rq_status_string(s: int) -> str:
    return load().rq_status_string(s).decode()


# ----------------------------------------------------------------------------- tensor wrappers
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return RQ_F32
    if t.dtype == torch.float16:
        return RQ_F16
    if t.dtype == torch.bfloat16:
        return RQ_BF16
    raise TypeError("unsupported dtype %s" % t.dtype)


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_2d(t, name, dtypes):
    """t is a contiguous 2-D tensor of one of `dtypes` (checked before any device access)."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D, got shape %s" % (name, tuple(t.shape)))
    if t.dtype not in dtypes:
        raise ValueError("%s dtype %s (expected one of %s)" % (name, t.dtype, ", ".join(map(str, dtypes))))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_vec(t, name, n):
    """t is a contiguous float32 vector of n elements (the C ABI reads exactly n floats)."""
    torch = _torch()
    if t.dtype != torch.float32 or t.dim() != 1 or t.shape[0] != n or not t.is_contiguous():
        raise ValueError("%s must be a contiguous float32 vector of %d elements, got %s %s"
                         % (name, n, t.dtype, tuple(t.shape)))


def _check_bytes(t, name, need, exact):
    """The C ABI sizes its buffer descriptors from the shapes, not from the allocation: the
    buffer must hold exactly (or, for outputs and scratch, at least) `need` bytes."""
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    nb = _nbytes(t)
    if nb < need or (exact and need > 0 and nb != need):
        raise ValueError("%s holds %d bytes, %s %d" % (name, nb, "expected" if exact else "needs at least", need))


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError("tensors are on different devices: %s" % sorted(map(str, devs)))


def code_shape(rows: int, K: int, bits: int) -> Tuple[int, int]:
    return (rows, K if bits == 8 else K // 2)


def workspace_size(M: int, K: int, bits: int = 8, w_layout: int = RQ_W_ROWS) -> int:
    return rq_rotq_linear_workspace_size(M, K, make_cfg(bits, w_layout=w_layout))


def quantize_weights(W, bits: int = 8, rot: int = 128, stream=None, w_scale_mode: int = RQ_W_ABSMAX,
                     w_layout: int = RQ_W_ROWS):
    """Offline: W [N, K] (f32/f16/bf16, device) -> (Wq, w_scale f32 [N]). Wq is int8 [N, K] /
    uint8 [N, K/2] (RQ_W_ROWS) or a flat uint8 buffer of rq_weight_bytes() holding FP6 tiles
    (RQ_W_FP6, bits 4). w_scale_mode: RQ_W_ABSMAX (per-row absmax), RQ_W_MSE (per-row
    MSE-optimized clipping) or RQ_W_TENSOR (one tensor-wise scale)."""
    torch = _torch()
    _check_2d(W, "W", (torch.float32, torch.float16, torch.bfloat16))
    N, K = W.shape
    cfg = make_cfg(bits, rot, w_scale_mode=w_scale_mode, w_layout=w_layout)
    if w_layout == RQ_W_ROWS:
        Wq = torch.empty(code_shape(N, K, bits), dtype=torch.int8 if bits == 8 else torch.uint8, device=W.device)
    else:
        Wq = torch.empty((max(rq_weight_bytes(N, K, cfg), 1),), dtype=torch.uint8, device=W.device)
    ws = torch.empty((N,), dtype=torch.float32, device=W.device)
    _check(rq_quantize_weights(_dev(W, "W"), _dtype_code(W), N, K, cfg,
                               Wq.data_ptr(), ws.data_ptr(), _stream(stream)), "rq_quantize_weights")
    return Wq, ws


def rotate_quantize(X, bits: int = 8, rot: int = 128, stream=None, x_layout: int = RQ_X_ROWS):
    """Online step alone: X [M, K] -> (Xq, x_scale f32 [M]). Xq is [M, K] int8 / [M, K/2] uint8
    (RQ_X_ROWS) or a flat uint8 buffer of rq_codes_bytes() in the tiled layout (RQ_X_TILED) or
    as FP6 tiles (RQ_X_FP6, bits 4)."""
    torch = _torch()
    _check_2d(X, "X", (torch.float32, torch.float16, torch.bfloat16))
    M, K = X.shape
    cfg = make_cfg(bits, rot, x_layout=x_layout)
    if x_layout == RQ_X_ROWS:
        Xq = torch.empty(code_shape(M, K, bits), dtype=torch.int8 if bits == 8 else torch.uint8, device=X.device)
    else:
        Xq = torch.empty((max(rq_codes_bytes(M, K, cfg), 1),), dtype=torch.uint8, device=X.device)
    xs = torch.empty((M,), dtype=torch.float32, device=X.device)
    _check(rq_rotate_quantize(_dev(X, "X"), _dtype_code(X), M, K, cfg,
                              Xq.data_ptr(), xs.data_ptr(), _stream(stream)), "rq_rotate_quantize")
    return Xq, xs


def _check_weights(Wq, w_scale, bias, N, K, cfg):
    _check_vec(w_scale, "w_scale", N)
    if bias is not None:
        _check_vec(bias, "bias", N)
    _check_bytes(Wq, "Wq", rq_weight_bytes(N, K, cfg), exact=True)


def rotq_linear(X, Wq, w_scale, bias=None, bits: int = 8, rot: int = 128, workspace=None,
                out=None, stream=None, w_layout: int = RQ_W_ROWS, act: int = RQ_ACT_NONE):
    """Y [M, N] = act(dequant(int GEMM(rotate+quantize(X), Wq)) + bias), in X's dtype;
    N = len(w_scale). w_layout must be the layout Wq was quantized in (RQ_W_FP6: the FP6
    matrix-core path); act is RQ_ACT_NONE, RQ_ACT_GELU_ERF or RQ_ACT_GELU_TANH. Shapes, dtypes
    and buffer sizes are checked here (ValueError) because the C ABI only sees pointers."""
    torch = _torch()
    _check_2d(X, "X", (torch.float16, torch.bfloat16))
    M, K = X.shape
    N = w_scale.shape[0] if w_scale.dim() == 1 else -1
    cfg = make_cfg(bits, rot, w_layout=w_layout, act=act)
    _check_weights(Wq, w_scale, bias, N, K, cfg)
    need = rq_rotq_linear_workspace_size(M, K, cfg)
    if workspace is not None:
        _check_bytes(workspace, "workspace", need, exact=False)
    if out is not None:
        if tuple(out.shape) != (M, N) or out.dtype != X.dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous %s tensor of shape (%d, %d), got %s %s"
                             % (X.dtype, M, N, out.dtype, tuple(out.shape)))
    _same_device(X, Wq, w_scale, bias, workspace, out)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=X.device)
    Y = torch.empty((M, N), dtype=X.dtype, device=X.device) if out is None else out
    _check(rq_rotq_linear(_dev(X, "X"), _dtype_code(X), M, K, _dev(Wq, "Wq"), _dev(w_scale, "w_scale"),
                          N, _dev(bias, "bias") if bias is not None else None, cfg, _dev(Y, "Y"),
                          _dev(workspace, "workspace"), _nbytes(workspace), _stream(stream)),
           "rq_rotq_linear")
    return Y


def _gemm_k(Wq, bits, K):
    if K is not None:
        return K
    if Wq.dim() != 2:
        raise ValueError("give K for a flat Wq buffer (FP6 weight tiles)")
    return Wq.shape[1] if bits == 8 else 2 * Wq.shape[1]


def gemm_dequant(Xq, x_scale, Wq, w_scale, bias=None, bits: int = 8, K: Optional[int] = None,
                 out_dtype=None, stream=None, x_layout: int = RQ_X_ROWS, w_layout: int = RQ_W_ROWS,
                 act: int = RQ_ACT_NONE):
    """Y [M, N] from codes, after the epilogue activation act; M = len(x_scale),
    N = len(w_scale), K from Wq unless given (give K for FP6 weight tiles)."""
    torch = _torch()
    M = x_scale.shape[0] if x_scale.dim() == 1 else -1
    N = w_scale.shape[0] if w_scale.dim() == 1 else -1
    K = _gemm_k(Wq, bits, K)
    cfg = make_cfg(bits, x_layout=x_layout, w_layout=w_layout, act=act)
    _check_vec(x_scale, "x_scale", M)
    _check_weights(Wq, w_scale, bias, N, K, cfg)
    _check_bytes(Xq, "Xq", rq_codes_bytes(M, K, cfg), exact=False)
    out_dtype = torch.float16 if out_dtype is None else out_dtype
    if out_dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("out_dtype must be float16 or bfloat16")
    _same_device(Xq, x_scale, Wq, w_scale, bias)
    Y = torch.empty((M, N), dtype=out_dtype, device=Xq.device)
    _check(rq_gemm_dequant(_dev(Xq, "Xq"), _dev(x_scale, "x_scale"), _dev(Wq, "Wq"), _dev(w_scale, "w_scale"),
                           _dev(bias, "bias") if bias is not None else None, M, N, K, cfg, Y.data_ptr(),
                           _dtype_code(Y), _stream(stream)), "rq_gemm_dequant")
    return Y


def gemm_s32(Xq, Wq, bits: int = 8, K: Optional[int] = None, stream=None,
             x_layout: int = RQ_X_ROWS, M: Optional[int] = None, N: Optional[int] = None,
             w_layout: int = RQ_W_ROWS):
    """acc [M, N] int32; M = Xq.shape[0] and N = Wq.shape[0] for row-major codes (give M for the
    tiled layouts, N and K for FP6 weight tiles)."""
    torch = _torch()
    if M is None:
        if x_layout != RQ_X_ROWS or Xq.dim() != 2:
            raise ValueError("give M for codes in a tiled layout")
        M = Xq.shape[0]
    if N is None:
        if w_layout != RQ_W_ROWS or Wq.dim() != 2:
            raise ValueError("give N for FP6 weight tiles")
        N = Wq.shape[0]
    K = _gemm_k(Wq, bits, K)
    cfg = make_cfg(bits, x_layout=x_layout, w_layout=w_layout)
    _check_bytes(Xq, "Xq", rq_codes_bytes(M, K, cfg), exact=False)
    _check_bytes(Wq, "Wq", rq_weight_bytes(N, K, cfg), exact=True)
    _same_device(Xq, Wq)
    acc = torch.empty((M, N), dtype=torch.int32, device=Xq.device)
    _check(rq_gemm_s32(_dev(Xq, "Xq"), _dev(Wq, "Wq"), M, N, K, cfg, acc.data_ptr(), _stream(stream)),
           "rq_gemm_s32")
    return acc
