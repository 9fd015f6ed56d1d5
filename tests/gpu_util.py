"""Helpers shared by the GPU parity tests (data movement only; no arithmetic of the method)."""
import numpy as np
import pytest
import torch

import oracle

IO_CODE = {"f16": oracle.F16, "bf16": oracle.BF16, "f32": oracle.F32}
TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def dev_from_bits(bits: np.ndarray, io: str) -> torch.Tensor:
    """uint16 raw bits (f16/bf16) or float32 array -> contiguous device tensor of that dtype."""
    if io == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits, np.float32)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DT[io]).cuda()


def bits_from_dev(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def codes_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    return t.numpy() if t.dtype == torch.int8 else t.numpy().view(np.uint8)


def boundary_mask(pre: np.ndarray) -> np.ndarray:
    """Codes whose pre-rounding value lies within one binary32 ulp of a .5 boundary."""
    p = pre.astype(np.float64)
    ulp = np.spacing(np.abs(pre).astype(np.float32)).astype(np.float64)
    return np.abs(p - (np.floor(p) + 0.5)) <= ulp


def compare_codes(gpu_codes, ref_codes, ref_pre, bits, K):
    """Bit-exact code comparison with the boundary exemption (<= 1e-5 of codes, each within one
    ulp of a .5 boundary). Returns (mismatches, exempt)."""
    g = gpu_codes if bits == 8 else oracle.unpack_int4(gpu_codes, K)
    diff = g != ref_codes
    n = int(diff.sum())
    if n:
        near = boundary_mask(ref_pre)
        assert np.all(near[diff]), "code mismatch away from a rounding boundary"
        assert n <= 1e-5 * diff.size, "too many boundary mismatches: %d of %d" % (n, diff.size)
        assert np.all(np.abs(g[diff].astype(int) - ref_codes[diff].astype(int)) == 1)
    return n


def y_tolerance_ok(y_gpu_bits, y_ref_bits, io):
    """max |err| <= 1e-3 + 2^-9 |ref| on the decoded outputs."""
    dt = IO_CODE[io]
    a = oracle.bits_to_f32(y_gpu_bits, dt).astype(np.float64)
    b = oracle.bits_to_f32(y_ref_bits, dt).astype(np.float64)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    err = np.abs(a[fin] - b[fin])
    return bool(np.all(err <= 1e-3 + 2.0**-9 * np.abs(b[fin]))), float(err.max(initial=0.0))


def _tiled_index(M, Kb):
    """For the tiled activation-code layout ([256-row panel][64-byte k step][256 rows][64 B],
    rows padded to whole panels), the flat byte index of every (row, byte) of an [M, Kb] array."""
    m = np.arange(M, dtype=np.int64)[:, None]
    b = np.arange(Kb, dtype=np.int64)[None, :]
    return (((m // 256) * (Kb // 64) + b // 64) * 256 + m % 256) * 64 + b % 64


def untile_codes(flat: np.ndarray, M: int, K: int, bits: int) -> np.ndarray:
    """Tiled code bytes -> row-major [M, Kb] (int8 for 8-bit, uint8 packed for 4-bit)."""
    Kb = K if bits == 8 else K // 2
    out = np.asarray(flat).view(np.uint8)[_tiled_index(M, Kb)]
    return out.view(np.int8) if bits == 8 else out


def tile_codes(rowmajor: np.ndarray, M: int, K: int, bits: int, pad_fill: int = 0x5A) -> np.ndarray:
    """Row-major code bytes [M, Kb] -> tiled flat buffer; pad rows get `pad_fill`."""
    Kb = K if bits == 8 else K // 2
    Mp = (M + 255) // 256 * 256
    out = np.full(Mp * Kb, pad_fill, dtype=np.uint8)
    out[_tiled_index(M, Kb)] = np.ascontiguousarray(rowmajor).view(np.uint8).reshape(M, Kb)
    return out
