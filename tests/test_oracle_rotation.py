"""Pins for the oracle's block-128 Walsh-Hadamard rotation.

The rotation is the "block-Hadamard ConvRot transform" of the SAM 3.1 release page
(section "Quantization recipe", step 2) and the "grouped, normalized Hadamard rotation" of the
TRELLIS.2 guide (section "What ConvRot changes"). Block size 128, Sylvester order and no sign
flips are readings (the pages fix none of them). Pins: the Sylvester matrix of a library
routine, orthogonality, the rotation-invariance identity, closed forms and an fp32 error bound.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle

H = scipy.linalg.hadamard(128).astype(np.float64)


def test_hadamard_entries_are_sylvester():
    ent = np.array([[oracle.hadamard_entry(i, j) for j in range(128)] for i in range(128)])
    assert np.array_equal(ent, H)


def test_fwht_of_unit_vectors_gives_hadamard_rows():
    E = np.eye(128, dtype=np.float32)
    U = oracle.fwht128_f32(E)            # row j = FWHT(e_j)
    assert np.array_equal(U.astype(np.float64), H)   # H is symmetric: FWHT(e_j) = H e_j


def test_fwht_of_ones():
    u = oracle.fwht128_f32(np.ones((1, 128), np.float32))[0]
    expect = np.zeros(128)
    expect[0] = 128
    assert np.array_equal(u, expect)


def test_fwht_involution_exact_on_integers():
    rng = np.random.default_rng(5)
    x = rng.integers(-1000, 1000, (4, 256)).astype(np.float32)
    y = oracle.fwht128_f32(oracle.fwht128_f32(x))
    assert np.array_equal(y, 128 * x)


def test_inv_sqrt_block_is_nearest_binary32():
    c = oracle.inv_sqrt_block()
    lo = np.nextafter(c, np.float32(0))
    hi = np.nextafter(c, np.float32(1))
    target_sq = Fraction(1, 128)
    mid_lo = (Fraction(float(lo)) + Fraction(float(c))) / 2
    mid_hi = (Fraction(float(c)) + Fraction(float(hi))) / 2
    assert mid_lo * mid_lo < target_sq < mid_hi * mid_hi
    assert c.view(np.uint32) == 0x3DB504F3


def test_rotation_is_orthogonal():
    R = oracle.rotate_f64(np.eye(256))            # rows of I -> rows of R (two blocks)
    assert np.abs(R @ R.T - np.eye(256)).max() < 1e-14
    assert np.abs(R - R.T).max() == 0.0           # symmetric, so R = R^T = R^-1
    R32 = R.astype(np.float32)
    err32 = np.abs(R32.astype(np.float64) @ R32.T.astype(np.float64) - np.eye(256)).max()
    assert err32 < 1e-6
    # block structure: no mixing across 128-blocks
    assert np.abs(R[:128, 128:]).max() == 0.0 and np.abs(R[128:, :128]).max() == 0.0


@pytest.mark.parametrize("M,N,K,seed", [(3, 5, 128, 0), (7, 4, 384, 1), (16, 33, 1024, 2)])
def test_rotation_invariance_fp64(M, N, K, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, 3, replace=False)] *= 50
    W = rng.normal(0, 0.02, (N, K))
    lhs = oracle.rotate_f64(X) @ oracle.rotate_f64(W).T
    rhs = X @ W.T
    assert np.abs(lhs - rhs).max() <= 1e-9 * np.abs(rhs).max()


def test_outlier_spreads_over_its_block():
    # A one-hot outlier a*e_c maps to magnitude |a|/sqrt(128) on every channel of its block and
    # to zero elsewhere: the "spread channel outliers" effect, in closed form.
    K, c, a = 512, 200, 37.5
    x = np.zeros((1, K))
    x[0, c] = a
    y = oracle.rotate_f64(x)[0]
    blk = c // 128
    inside = y[blk * 128:(blk + 1) * 128]
    assert np.allclose(np.abs(inside), a / np.sqrt(128), rtol=0, atol=1e-12)
    assert np.abs(np.delete(y, np.arange(blk * 128, (blk + 1) * 128))).max() == 0.0
    # the signs follow column c % 128 of the Sylvester matrix
    assert np.array_equal(np.sign(inside), H[c % 128])


def test_fwht_f32_within_error_bound_of_exact():
    # f16 inputs: each value is an integer times 2^-24 below 2^16, so fp64 sums of 128 terms
    # are exact; fp32 butterflies over 7 stages err by at most gamma_7 * sum|x| per output.
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 1024)) * 3).astype(np.float16).astype(np.float32)
    x[:, 7] *= 50
    x = x.astype(np.float16).astype(np.float32)
    u32 = oracle.fwht128_f32(x).astype(np.float64)
    xb = x.astype(np.float64).reshape(64, 8, 128)
    exact = np.einsum("rbi,ij->rbj", xb, H).reshape(64, 1024)
    gamma7 = 7 * 2.0**-24 / (1 - 7 * 2.0**-24)
    bound = gamma7 * np.repeat(np.abs(xb).sum(-1), 128, axis=1)
    assert np.all(np.abs(u32 - exact) <= bound)
    assert np.count_nonzero(u32 != exact) > 0  # the bound is exercised, not vacuous


def test_fwht_f32_times_c_matches_rotation():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    c = float(oracle.inv_sqrt_block())
    got = oracle.fwht128_f32(x).astype(np.float64) * c
    ref = oracle.rotate_f64(x.astype(np.float64))
    assert np.abs(got - ref).max() < 1e-5 * np.abs(ref).max()


def test_fwht_stage_order_golden():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fwht_stage_order.json")))
    x = np.zeros((1, 128), np.float32)
    for k, v in g["x"].items():
        x[0, int(k)] = v
    u = oracle.fwht128_f32(x)[0]
    for k, v in g["out"].items():
        assert float(u[int(k)]) == v
