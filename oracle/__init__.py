"""CPU oracle for the ConvRot quantized linear (rotate -> per-row quantize -> int GEMM -> dequant).

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never touches it, and the two share no code.

The arithmetic lives in ``convrot_oracle.c`` (plain C, one correctly rounded fp32 operation
per step); this module only marshals numpy arrays through ctypes and composes the steps in the
order the method applies them:

* "SAM 3.1 Multiplex INT8/INT4 ConvRot" page, section "Quantization recipe": FP32 upcast,
  block-Hadamard ConvRot transform, per-row scales; online activation quantization (W8A8 / W4A4).
* "TRELLIS.2 INT8 ConvRot in ComfyUI" guide, section "What ConvRot changes": grouped,
  normalized Hadamard rotation before per-row weight quantization, the matching rotation on
  activations at run time.

fp64 shadows (``rotate_f64``, ``linear_f64``) are reporting and pinning aids, not the spec.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

F32, F16, BF16 = 0, 1, 2
BLOCK = 128

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.orc_quantize_rows.argtypes = [P, I, I64, I64, I, I, P, P, P]
        lib.orc_quantize_rows.restype = I
        lib.orc_pack_int4.argtypes = [P, I64, I64, P]
        lib.orc_unpack_int4.argtypes = [P, I64, I64, P]
        lib.orc_gemm_s32.argtypes = [P, P, I64, I64, I64, P]
        lib.orc_gemm_s32.restype = I
        lib.orc_epilogue.argtypes = [P, P, P, P, I64, I64, I, P]
        lib.orc_epilogue_act.argtypes = [P, P, P, P, I64, I64, I, I, P, P]
        lib.orc_gelu_f64_array.argtypes = [P, I64, I, P]
        lib.orc_rotate_f64.argtypes = [P, I64, I64, P]
        for name in ("orc_f32_to_f16_array", "orc_f32_to_bf16_array",
                     "orc_f16_to_f32_array", "orc_bf16_to_f32_array"):
            getattr(lib, name).argtypes = [P, I64, P]
        lib.orc_fwht128_rows.argtypes = [P, I64]
        lib.orc_inv_sqrt_block.restype = ctypes.c_float
        lib.orc_hadamard_entry.argtypes = [I, I]
        lib.orc_hadamard_entry.restype = I
        lib.orc_num_threads.restype = I
        lib.orc_set_num_threads.argtypes = [I]
        lib.orc_quantize_rows_mse.argtypes = [P, I, I64, I64, I, P, P, P, P]
        lib.orc_quantize_rows_mse.restype = I
        lib.orc_quantize_tensorwise.argtypes = [P, I, I64, I64, I, P, P, P]
        lib.orc_quantize_tensorwise.restype = I
        lib.orc_clip_alpha.argtypes = [I]
        lib.orc_clip_alpha.restype = ctypes.c_float
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def num_threads() -> int:
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads the oracle's OpenMP loops use from now on (timing runs only)."""
    _load().orc_set_num_threads(int(n))


# ---------------------------------------------------------------------------- formats
def f32_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    _load().orc_f32_to_f16_array(_ptr(x), x.size, _ptr(y))
    return y


def f32_to_bf16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    _load().orc_f32_to_bf16_array(_ptr(x), x.size, _ptr(y))
    return y


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    y = np.empty(h.shape, np.float32)
    _load().orc_f16_to_f32_array(_ptr(h), h.size, _ptr(y))
    return y


def bf16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    y = np.empty(h.shape, np.float32)
    _load().orc_bf16_to_f32_array(_ptr(h), h.size, _ptr(y))
    return y


def bits_to_f32(x: np.ndarray, dtype: int) -> np.ndarray:
    """Exact upcast of f32 / f16-bits / bf16-bits arrays to float32."""
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    return f16_bits_to_f32(x) if dtype == F16 else bf16_bits_to_f32(x)


# ---------------------------------------------------------------------------- rotation
def inv_sqrt_block() -> np.float32:
    return np.float32(_load().orc_inv_sqrt_block())


def hadamard_entry(i: int, j: int) -> int:
    return _load().orc_hadamard_entry(i, j)


def fwht128_f32(v) -> np.ndarray:
    """Unnormalized fp32 FWHT of every 128-block of the last axis (returns a copy)."""
    v = np.array(v, dtype=np.float32, copy=True, order="C")
    assert v.shape[-1] % BLOCK == 0
    _load().orc_fwht128_rows(_ptr(v), v.size // BLOCK)
    return v


def rotate_f64(x) -> np.ndarray:
    """fp64 x @ blockdiag(H_128/sqrt(128)) as an explicit matrix product per block."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    rows, K = x.reshape(-1, x.shape[-1]).shape
    y = np.empty_like(x)
    _load().orc_rotate_f64(_ptr(x), rows, K, _ptr(y))
    return y


# ---------------------------------------------------------------------------- quantizer
def quantize_rows(x: np.ndarray, dtype: int, bits: int = 8, rotate: bool = True,
                  want_pre: bool = False):
    """Rotate (optional) and quantize each row of x.

    x: [rows, K] float32 (dtype F32) or uint16 raw bits (F16 / BF16).
    Returns (codes int8 [rows, K] unpacked, scales float32 [rows], pre float32 [rows, K] or None).
    """
    x = np.ascontiguousarray(x)
    assert x.ndim == 2
    rows, K = x.shape
    if dtype == F32:
        assert x.dtype == np.float32
    else:
        assert x.dtype == np.uint16
    codes = np.empty((rows, K), np.int8)
    scales = np.empty((rows,), np.float32)
    pre = np.empty((rows, K), np.float32) if want_pre else None
    rc = _load().orc_quantize_rows(_ptr(x), dtype, rows, K, bits, 1 if rotate else 0,
                                   _ptr(codes), _ptr(scales),
                                   _ptr(pre) if pre is not None else None)
    if rc != 0:
        raise RuntimeError("oracle quantize_rows failed (%d)" % rc)
    return codes, scales, pre


NCLIP = 51   # clipping candidates alpha_i = fl((100 - i) / 100), i = 0..50


def clip_alpha(i: int) -> np.float32:
    return np.float32(_load().orc_clip_alpha(i))


def _check_rows_input(x, dtype):
    x = np.ascontiguousarray(x)
    assert x.ndim == 2
    if dtype == F32:
        assert x.dtype == np.float32
    else:
        assert x.dtype == np.uint16
    return x


def quantize_rows_mse(x: np.ndarray, dtype: int, bits: int = 8):
    """Rotate, then per-row MSE-optimized clipping (the release page's recipe, step 3).

    Returns (codes int8 [rows, K], scales float32 [rows], alpha_idx int32 [rows],
    err float64 [rows, NCLIP] -- every candidate's squared reconstruction error)."""
    x = _check_rows_input(x, dtype)
    rows, K = x.shape
    codes = np.empty((rows, K), np.int8)
    scales = np.empty((rows,), np.float32)
    idx = np.empty((rows,), np.int32)
    err = np.empty((rows, NCLIP), np.float64)
    rc = _load().orc_quantize_rows_mse(_ptr(x), dtype, rows, K, bits, _ptr(codes), _ptr(scales),
                                       _ptr(idx), _ptr(err))
    if rc != 0:
        raise RuntimeError("oracle quantize_rows_mse failed (%d)" % rc)
    return codes, scales, idx, err


def quantize_tensorwise(x: np.ndarray, dtype: int, bits: int = 8, want_pre: bool = False):
    """Rotate, then one absmax scale for the whole tensor (every row gets the same scale).

    Returns (codes int8 [rows, K], scales float32 [rows], pre float32 [rows, K] or None)."""
    x = _check_rows_input(x, dtype)
    rows, K = x.shape
    codes = np.empty((rows, K), np.int8)
    scales = np.empty((rows,), np.float32)
    pre = np.empty((rows, K), np.float32) if want_pre else None
    rc = _load().orc_quantize_tensorwise(_ptr(x), dtype, rows, K, bits, _ptr(codes), _ptr(scales),
                                         _ptr(pre) if pre is not None else None)
    if rc != 0:
        raise RuntimeError("oracle quantize_tensorwise failed (%d)" % rc)
    return codes, scales, pre


def pack_int4(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    rows, K = codes.shape
    out = np.empty((rows, K // 2), np.uint8)
    _load().orc_pack_int4(_ptr(codes), rows, K, _ptr(out))
    return out


def unpack_int4(packed: np.ndarray, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    out = np.empty((rows, K), np.int8)
    _load().orc_unpack_int4(_ptr(packed), rows, K, _ptr(out))
    return out


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Storage layout of the codes: int8 [rows, K] as is, int4 two per byte."""
    return np.ascontiguousarray(codes, dtype=np.int8) if bits == 8 else pack_int4(codes)


# ---------------------------------------------------------------------------- GEMM + epilogue
def gemm_s32(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k A[m, k] B[n, k] (exact, must fit int32)."""
    A = np.ascontiguousarray(A, dtype=np.int8)
    B = np.ascontiguousarray(B, dtype=np.int8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    acc = np.empty((M, N), np.int32)
    if _load().orc_gemm_s32(_ptr(A), _ptr(B), M, N, K, _ptr(acc)) != 0:
        raise OverflowError("int32 accumulator overflow")
    return acc


def epilogue(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray, bias, out_dtype: int) -> np.ndarray:
    """Y bits = cast(fma(f32(acc), s_w[n]*s_x[m], bias[n])) (uint16 raw bits)."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    sx = np.ascontiguousarray(sx, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, N = acc.shape
    assert sx.shape == (M,) and sw.shape == (N,)
    b = None
    if bias is not None:
        b = np.ascontiguousarray(bias, dtype=np.float32)
        assert b.shape == (N,)
    Y = np.empty((M, N), np.uint16)
    _load().orc_epilogue(_ptr(acc), _ptr(sx), _ptr(sw), _ptr(b) if b is not None else None,
                         M, N, out_dtype, _ptr(Y))
    return Y


ACT_NONE, ACT_GELU_ERF, ACT_GELU_TANH = 0, 1, 2


def gelu_f64(v: np.ndarray, act: int) -> np.ndarray:
    """GELU in binary64, element-wise (act 1: erf form, act 2: tanh form, 0: identity)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    g = np.empty_like(v)
    _load().orc_gelu_f64_array(_ptr(v), v.size, act, _ptr(g))
    return g


def epilogue_act(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray, bias, out_dtype: int, act: int):
    """The epilogue with the MLP activation fused: (Y bits, g64), where
    Y = cast(f32(GELU64(fma(f32(acc), s_w[n]*s_x[m], bias[n])))) and g64 is GELU64 before the
    two roundings (the value a one-ulp difference near a rounding midpoint is judged by)."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    sx = np.ascontiguousarray(sx, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, N = acc.shape
    assert sx.shape == (M,) and sw.shape == (N,)
    b = None
    if bias is not None:
        b = np.ascontiguousarray(bias, dtype=np.float32)
        assert b.shape == (N,)
    Y = np.empty((M, N), np.uint16)
    g = np.empty((M, N), np.float64)
    _load().orc_epilogue_act(_ptr(acc), _ptr(sx), _ptr(sw), _ptr(b) if b is not None else None,
                             M, N, act, out_dtype, _ptr(Y), _ptr(g))
    return Y, g


# ---------------------------------------------------------------------------- whole path
def quantize_weights(W: np.ndarray, bits: int = 8, rotate: bool = True, w_dtype: int = F32):
    """Offline step: (codes unpacked int8 [N, K], storage [N, K] or [N, K/2], w_scale [N])."""
    codes, scales, _ = quantize_rows(W, w_dtype, bits, rotate)
    return codes, pack_codes(codes, bits), scales


def rotq_linear(X: np.ndarray, x_dtype: int, W_codes: np.ndarray, w_scale: np.ndarray, bias,
                bits: int = 8, rotate: bool = True, act: int = ACT_NONE):
    """Online step on X bits [M, K] against already quantized weights.

    Returns dict with x_codes, x_scale, acc, Y (uint16 bits in X's dtype) and, with an
    activation, g64 (its binary64 value before rounding) and v (the fp32 pre-activation).
    """
    xc, xs, _ = quantize_rows(X, x_dtype, bits, rotate)
    acc = gemm_s32(xc, W_codes)
    out = {"x_codes": xc, "x_scale": xs, "acc": acc}
    if act == ACT_NONE:
        out["Y"] = epilogue(acc, xs, w_scale, bias, x_dtype)
    else:
        out["Y"], out["g64"] = epilogue_act(acc, xs, w_scale, bias, x_dtype, act)
        out["v"] = epilogue_act(acc, xs, w_scale, bias, x_dtype, ACT_NONE)[1]
    return out


def linear_f64(X: np.ndarray, W: np.ndarray, bias) -> np.ndarray:
    """Unquantized reference X W^T + bias in fp64 (quantization-error context only)."""
    Y = np.asarray(X, np.float64) @ np.asarray(W, np.float64).T
    if bias is not None:
        Y = Y + np.asarray(bias, np.float64)[None, :]
    return Y
