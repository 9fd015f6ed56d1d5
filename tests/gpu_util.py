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


# ---- FP6 tiles (4-bit codes stored as FP6 E2M3; layout documented in include/convrot.h) ----
_FP6_MAG = np.array([0, 8, 16, 20, 24, 26, 28, 30], np.uint8)


def _fp6_value_table() -> np.ndarray:
    """Value of every 6-bit E2M3 pattern (sign bit 5, exponent bits 4..3 with bias 1, mantissa
    bits 2..0; exponent 0 is subnormal: m / 8)."""
    v = np.zeros(64, np.float64)
    for p in range(64):
        e, m = (p >> 3) & 3, p & 7
        mag = m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1 + m / 8.0)
        v[p] = -mag if p & 32 else mag
    return v


_FP6_VALUE = _fp6_value_table()


def _fp6_index(rows: int, K: int, P: int):
    """Flat byte index of byte j (0..23) of the operand string of (row, slice, half), as arrays
    [rows, K/64, 2, 24]."""
    nsl = K // 64
    r = np.arange(rows, dtype=np.int64)[:, None, None, None]
    s = np.arange(nsl, dtype=np.int64)[None, :, None, None]
    h = np.arange(2, dtype=np.int64)[None, None, :, None]
    j = np.arange(24, dtype=np.int64)[None, None, None, :]
    base = ((r // P) * nsl + s) * (P * 48)
    rr = r % P
    p1 = base + rr * 32 + 16 * (h ^ ((rr >> 3) & 1)) + j
    p2 = base + P * 32 + rr * 16 + 8 * (h ^ ((rr >> 4) & 1)) + (j - 16)
    return np.where(j < 16, p1, p2)


def fp6_untile(flat: np.ndarray, rows: int, K: int, P: int) -> np.ndarray:
    """FP6 tiles -> int8 codes [rows, K] (every value must be an integer in [-7, 7])."""
    b = np.asarray(flat).view(np.uint8)[_fp6_index(rows, K, P)].astype(np.uint32)   # [rows, nsl, 2, 24]
    g = b[..., 0::3] | (b[..., 1::3] << 8) | (b[..., 2::3] << 16)                      # 8 fields of 24 bits
    pats = np.stack([(g >> (6 * i)) & 63 for i in range(4)], axis=-1)                 # [rows, nsl, 2, 8, 4]
    vals = _FP6_VALUE[pats.reshape(rows, K)]
    assert np.all(vals == np.rint(vals)) and np.all(np.abs(vals) <= 7)
    return vals.astype(np.int8)


def fp6_tile(codes: np.ndarray, P: int, pad_fill: int = 0x5A) -> np.ndarray:
    """int8 codes [rows, K] in [-7, 7] -> flat FP6 tiles (pad rows filled with pad_fill)."""
    rows, K = codes.shape
    c = codes.astype(np.int64)
    pats = (_FP6_MAG[np.abs(c)].astype(np.uint32) | np.where(c < 0, 32, 0).astype(np.uint32))
    pats = pats.reshape(rows, K // 64, 2, 8, 4)
    g = pats[..., 0] | (pats[..., 1] << 6) | (pats[..., 2] << 12) | (pats[..., 3] << 18)
    b = np.stack([g & 255, (g >> 8) & 255, (g >> 16) & 255], axis=-1).reshape(rows, K // 64, 2, 24)
    out = np.full((rows + P - 1) // P * P * (K // 64) * 48, pad_fill, np.uint8)
    out[_fp6_index(rows, K, P)] = b.astype(np.uint8)
    return out


def act_window(v, act):
    """Relative error bound of the GPU's binary32 GELU at pre-activation v, from the function's
    conditioning: a few binary32 ulps, plus the rounding of the inner argument amplified by the
    tail -- d ln(x Phi(x)) / dt ~ 2|t| with t = v / sqrt 2 (erf form), d ln(x logistic(2u)) / du
    ~ 2 with u = sqrt(2/pi) (v + 0.044715 v^3) (tanh form) -- with a factor of 4 to spare."""
    v = np.asarray(v, np.float64)
    if act == oracle.ACT_GELU_ERF:
        t = v / np.sqrt(2.0)
        return 2.0 ** -18 + t * t * 2.0 ** -19
    u = np.sqrt(2.0 / np.pi) * (v + 0.044715 * v ** 3)
    return 2.0 ** -18 + np.abs(u) * 2.0 ** -18


def act_outputs_match(y_gpu, y_ref, g64, out, v, act, max_frac=1e-3):
    """Outputs of an epilogue with a fused GELU against the oracle's: equal, except that an
    element may be the adjacent fp16/bf16 value when the oracle's binary64 GELU lies within
    act_window(v) (relative) of the midpoint between the two, or a zero where the exact value
    is below the binary32 normal range. Returns (ok, number of differing elements, detail)."""
    y_gpu = np.asarray(y_gpu, np.uint16)
    y_ref = np.asarray(y_ref, np.uint16)
    diff = y_gpu != y_ref
    n = int(diff.sum())
    if n == 0:
        return True, 0, ""
    a = oracle.bits_to_f32(y_gpu[diff], out).astype(np.float64)
    b = oracle.bits_to_f32(y_ref[diff], out).astype(np.float64)
    g = np.asarray(g64)[diff]
    w = act_window(np.asarray(v)[diff], act)
    # adjacent representable values: same sign and bit patterns one apart
    gi, ri = y_gpu[diff].astype(np.int32), y_ref[diff].astype(np.int32)
    adjacent = (((gi ^ ri) & 0x8000) == 0) & (np.abs(gi - ri) == 1)
    near_mid = np.abs(g - 0.5 * (a + b)) <= w * np.maximum(np.abs(g), 1e-300)
    # Below the binary32 normal range (2^-126) the native exp2 may flush its result to zero:
    # such values (bf16 subnormals; fp16 holds none of them) may come out as a signed zero.
    tiny = (np.abs(g) < 2.0 ** -126) & (np.minimum(np.abs(a), np.abs(b)) == 0) & \
        (np.maximum(np.abs(a), np.abs(b)) < 2.0 ** -126)
    exempt = (adjacent & near_mid) | tiny
    ok = bool(np.all(exempt)) and n <= max_frac * y_gpu.size
    bad = np.flatnonzero(~exempt)[:5]
    return ok, n, "%d differing of %d; first not exempt: gpu %s ref %s g64 %s v %s" % (
        n, y_gpu.size, a[bad], b[bad], g[bad], np.asarray(v)[diff][bad])
