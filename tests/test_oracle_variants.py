"""Pins for the oracle's two weight-quantizer variants.

MSE-optimized clipping: 'SAM 3.1 Multiplex INT8/INT4 ConvRot' page, 'Quantization recipe', step 3
(after the block-Hadamard transform the converter picks a clipping scale that minimizes the
squared error). The page fixes neither the candidate grid nor the tie rule; the oracle searches
alpha = 1.00, 0.99, ..., 0.50 of the row's absmax and keeps the larger alpha on a tie.

Tensor-wise scale: the HSWQ ConvRot model card ('int8_tensorwise') and the 'Explanation of INT8
ConvRot' taxonomy table (scaling method: none / tensor-wise / row-wise). One absmax over the
whole rotated tensor, shared by every row.

Expected values come from exact rational arithmetic, closed forms for uniform data, or the
already pinned absmax quantizer -- never from the function under test.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
from tests.exact import f32_nearest

H = scipy.linalg.hadamard(128).astype(np.float64)


def _c32():
    """fl(1/sqrt(128)) = fl(2^-3.5), from exact rationals: the binary32 nearest to 1/sqrt(128)."""
    c = np.float32(1 / np.sqrt(128.0))
    # Check against the defining property |c^2 * 128 - 1| minimal among neighbours.
    cands = [np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(1))]
    return min(cands, key=lambda v: abs(Fraction(float(v)) ** 2 * 128 - 1))


C32 = _c32()


def _x_with_rotation(u):
    """Rows x with FWHT(x) = u: x = H u / 128 per 128-block, exact when u holds small integers."""
    u = np.asarray(u, np.float64)
    x = np.empty_like(u)
    for b in range(u.shape[1] // 128):
        x[:, b * 128:(b + 1) * 128] = u[:, b * 128:(b + 1) * 128] @ H.T / 128.0
    return x


def _exact_err(u32, s, q):
    """sum_k (u_k c - s q_k)^2 in exact rationals."""
    c, sf = Fraction(float(C32)), Fraction(float(s))
    return sum((Fraction(float(v)) * c - sf * int(k)) ** 2 for v, k in zip(u32, q))


def _candidate(u32, a, i, qmax):
    """Candidate i on the pages' step order, each binary32 operation correctly rounded
    (numpy's float32 arithmetic is IEEE): t = fl(a*alpha), inv = fl(qmax/t), s = fl(fl(t c)/qmax),
    q = clamp(rne(fl(u inv)))."""
    alpha = f32_nearest(Fraction(100 - i, 100))
    t = np.float32(a) * alpha
    inv = np.float32(qmax) / t
    s = (t * C32) / np.float32(qmax)
    q = np.clip(np.rint(u32 * inv), -qmax, qmax).astype(np.int64)
    return s, q


def test_clip_alpha_grid():
    assert oracle.NCLIP == 51
    for i in range(oracle.NCLIP):
        assert oracle.clip_alpha(i) == f32_nearest(Fraction(100 - i, 100))


@pytest.mark.parametrize("bits,seed", [(4, 0), (4, 1), (8, 2)])
def test_mse_clip_brute_force_exact(bits, seed):
    """Every candidate's error in exact rationals, then the argmin (smallest index on a tie)."""
    rng = np.random.default_rng(seed)
    qmax = 127 if bits == 8 else 7
    rows, K = 4, 128
    u = rng.integers(-40, 41, (rows, K)).astype(np.float64)
    u[0, 7] = 400                                  # one outlier: clipping it pays
    u[1] = rng.integers(-3, 4, K) * 30             # few distinct magnitudes
    x = _x_with_rotation(u).astype(np.float32)
    assert np.array_equal(oracle.fwht128_f32(x).astype(np.float64), u)   # rotation exact
    codes, scales, idx, err = oracle.quantize_rows_mse(x, oracle.F32, bits)
    for r in range(rows):
        u32 = u[r].astype(np.float32)
        a = np.abs(u32).max()
        exact = []
        for i in range(oracle.NCLIP):
            s, q = _candidate(u32, a, i, qmax)
            exact.append(_exact_err(u32, s, q))
        for i in range(oracle.NCLIP):       # the oracle's binary64 sums: a few ulps off
            assert abs(err[r, i] - float(exact[i])) <= 1e-12 * float(exact[i]) + 1e-300
        best = min(range(oracle.NCLIP), key=lambda i: (exact[i], i))
        second = min((exact[i] for i in range(oracle.NCLIP) if exact[i] != exact[best]),
                     default=exact[best])
        if float(second - exact[best]) > 1e-9 * float(exact[best]):
            assert idx[r] == best, (r, idx[r], best)
        s, q = _candidate(u32, a, int(idx[r]), qmax)
        assert scales[r] == s
        assert np.array_equal(codes[r].astype(np.int64), q)
    if bits == 4:
        assert idx[0] > 0                      # the outlier row clips at 4 bits


def test_mse_clip_constant_magnitude_row_keeps_absmax():
    """|u_k| all equal: any alpha < 1 clamps every code and adds K((1-alpha) a c)^2, so
    alpha = 1 wins and the result equals the absmax quantizer's."""
    u = np.where(np.arange(256) % 3 == 0, 5.0, -5.0)[None, :]
    x = _x_with_rotation(u).astype(np.float32)
    for bits in (8, 4):
        codes, scales, idx, err = oracle.quantize_rows_mse(x, oracle.F32, bits)
        c0, s0, _ = oracle.quantize_rows(x, oracle.F32, bits)
        assert idx[0] == 0
        assert np.array_equal(codes, c0) and np.array_equal(scales, s0)
        assert np.all(err[0, 1:] > err[0, 0])


@pytest.mark.parametrize("bits", [8, 4])
def test_mse_clip_absmax_candidate_and_choice_consistent(bits):
    """err[:, 0] is the absmax quantizer's error; the returned codes/scale realize err[idx],
    which is the minimum of the row's err (first index among equals)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 384)).astype(np.float32)
    x[:, rng.choice(384, 3, replace=False)] *= 30
    codes, scales, idx, err = oracle.quantize_rows_mse(x, oracle.F32, bits)
    c0, s0, _ = oracle.quantize_rows(x, oracle.F32, bits)
    u = oracle.fwht128_f32(x)
    for r in range(6):
        e0 = _exact_err(u[r], s0[r], c0[r])
        assert abs(err[r, 0] - float(e0)) <= 1e-12 * float(e0)
        e = _exact_err(u[r], scales[r], codes[r])
        assert abs(err[r, idx[r]] - float(e)) <= 1e-12 * float(e)
        assert idx[r] == int(np.argmin(err[r]))   # argmin returns the first minimum
        assert err[r, idx[r]] <= err[r, 0]
        if idx[r] == 0:
            assert np.array_equal(codes[r], c0[r]) and scales[r] == s0[r]


def test_mse_clip_uniform_data_closed_form():
    """Uniform data on [-a, a]: the squared error is smallest when the 2 q_max + 1 levels sit at
    the centres of equal cells, step 2a/(2 q_max + 1), i.e. alpha* = 2 q_max / (2 q_max + 1)
    (14/15 = 0.933 at 4 bits). A long row's sample optimum lands next to it."""
    rng = np.random.default_rng(8)
    K = 32768
    u = rng.uniform(-1.0, 1.0, (3, K))
    u[:, 0] = 1.0
    x = _x_with_rotation(u).astype(np.float32)
    _, _, idx, _ = oracle.quantize_rows_mse(x, oracle.F32, 4)
    alphas = [(100 - int(i)) / 100 for i in idx]
    assert all(0.92 <= al <= 0.95 for al in alphas), alphas
    _, _, idx8, _ = oracle.quantize_rows_mse(x, oracle.F32, 8)
    assert all(int(i) <= 1 for i in idx8)      # alpha* = 254/255 = 0.996


def test_mse_clip_gaussian_int4_clips_and_helps():
    """Heavy clipping pays for bell-shaped rows at 4 bits: the chosen alpha is well below 1 and
    the error against the exact rotated row drops."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 1024)).astype(np.float32)
    codes, scales, idx, _ = oracle.quantize_rows_mse(x, oracle.F32, 4)
    c0, s0, _ = oracle.quantize_rows(x, oracle.F32, 4)
    y = oracle.rotate_f64(x.astype(np.float64))
    e_mse = np.linalg.norm(codes * scales[:, None].astype(np.float64) - y)
    e_abs = np.linalg.norm(c0 * s0[:, None].astype(np.float64) - y)
    assert np.all(idx >= 15)                   # alpha <= 0.85
    assert e_mse < 0.85 * e_abs


def test_mse_clip_zero_row_and_f16_input():
    x = np.zeros((2, 256), np.float16)
    x[1, 3] = 2.0
    codes, scales, idx, err = oracle.quantize_rows_mse(x.view(np.uint16), oracle.F16, 8)
    assert scales[0] == 0 and not codes[0].any() and idx[0] == 0 and not err[0].any()
    c0, s0, _ = oracle.quantize_rows(x.view(np.uint16)[1:], oracle.F16, 8)
    assert idx[1] == 0                        # |u| constant over the first block, 0 elsewhere
    assert np.array_equal(codes[1:], c0) and scales[1] == s0[0]


# ---- tensor-wise -------------------------------------------------------------------------


def test_tensorwise_single_row_is_rowwise():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 512)).astype(np.float32)
    for bits in (8, 4):
        c, s, _ = oracle.quantize_tensorwise(x, oracle.F32, bits)
        c0, s0, _ = oracle.quantize_rows(x, oracle.F32, bits)
        assert np.array_equal(c, c0) and np.array_equal(s, s0)


@pytest.mark.parametrize("bits", [8, 4])
def test_tensorwise_exact(bits):
    """One scale fl(fl(A c)/q_max) for all rows, A = max |u| over the tensor; codes are the
    nearest integers of u q_max / A in exact rationals (away from .5 boundaries)."""
    rng = np.random.default_rng(6 + bits)
    qmax = 127 if bits == 8 else 7
    u = rng.integers(-60, 61, (5, 256)).astype(np.float64)
    u[3, 100] = -900
    u[4] *= 0                                  # a zero row shares the tensor's scale
    x = _x_with_rotation(u).astype(np.float32)
    codes, scales, pre = oracle.quantize_tensorwise(x, oracle.F32, bits, want_pre=True)
    A = Fraction(900)
    s = f32_nearest(Fraction(float(f32_nearest(A * Fraction(float(C32))))) / qmax)
    assert np.all(scales == s)
    inv = f32_nearest(Fraction(qmax) / A)
    for r in range(5):
        for k in range(256):
            p = f32_nearest(Fraction(int(u[r, k])) * Fraction(float(inv)))
            assert pre[r, k] == p
            t = Fraction(int(u[r, k]) * qmax, 900)
            fl = t.__floor__()
            if abs(t - (fl + Fraction(1, 2))) > Fraction(1, 1000):
                assert codes[r, k] == round(t)
    assert codes[3, 100] == -qmax and not codes[4].any()
    assert np.abs(codes[:3]).max() < qmax      # only the tensor's absmax reaches the edge


def test_tensorwise_zero_tensor():
    c, s, _ = oracle.quantize_tensorwise(np.zeros((3, 128), np.float32), oracle.F32, 8)
    assert not c.any() and not s.any()


def test_mse_clip_candidates_with_overflowing_reciprocal_are_zero_rows():
    """Near the reciprocal-overflow edge some clipping candidates t_i = fl(a alpha_i) have an
    infinite fl(q_max / t_i): each quantizes the row to zero, so its error is the row's own
    energy sum_k (u_k c)^2 (binary64, increasing k), and the choice still follows the errors.
    A row whose a itself overflows is a zero row (scale 0, codes 0)."""
    from tests.test_oracle_quant import _inv_overflow_edge
    qmax = 127
    a_lo, _ = _inv_overflow_edge(qmax)
    a = np.float32(a_lo * np.float32(1.5))            # alpha = 1 finite; alpha <= 2/3 overflow
    x = np.zeros((2, 128), np.float32)
    x[0, 0] = a
    x[1, 0] = a_lo
    codes, scales, idx, err = oracle.quantize_rows_mse(x, oracle.F32, 8)
    c = float(C32)
    energy = 0.0
    for k in range(128):
        d = float(a) * c - 0.0
        energy += d * d
    zero_cands = [i for i in range(51) if np.isinf(np.float32(qmax) / np.float32(a * oracle.clip_alpha(i)))]
    assert zero_cands and zero_cands[0] > 0
    for i in zero_cands:
        assert err[0, i] == energy
    assert idx[0] == 0 and np.all(codes[0] == qmax)   # constant |u|: alpha = 1 has no error
    assert scales[1] == 0 and not codes[1].any()


def test_tensorwise_reciprocal_overflow_is_zero_tensor():
    from tests.test_oracle_quant import _inv_overflow_edge
    a_lo, a_hi = _inv_overflow_edge(7)
    x = np.zeros((3, 128), np.float32)
    x[1, 0] = a_lo
    c, s, _ = oracle.quantize_tensorwise(x, oracle.F32, 4)
    assert not c.any() and not s.any()
    x[2, 0] = a_hi
    c, s, _ = oracle.quantize_tensorwise(x, oracle.F32, 4)
    assert np.all(s == s[0]) and s[0] > 0 and np.all(c[2] == 7)
