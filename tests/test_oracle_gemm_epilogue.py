"""Pins for the oracle's integer GEMM and dequantizing epilogue.

Passages: 'SAM 3.1 Multiplex INT8/INT4 ConvRot' page, 'Quantization recipe' (W8A8 / W4A4
operations, per-row scales) and 'Downloads' (INT4 products may run as INT8 multiplication);
'HSWQ ConvRot INT8' card (INT8 tensor-core operations). The int32 accumulator is a plain
definition, pinned by brute force with Python integers; the epilogue by hand-derived cases
and by an exact-rational fused multiply-add.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact import f32_nearest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 128, 0), (3, 5, 128, 1), (9, 17, 256, 2), (4, 16, 384, 3)])
def test_gemm_bruteforce_python_ints(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = rng.integers(-127, 128, (M, K)).astype(np.int8)
    B = rng.integers(-127, 128, (N, K)).astype(np.int8)
    acc = oracle.gemm_s32(A, B)
    for m in range(M):
        for n in range(N):
            assert int(acc[m, n]) == sum(int(a) * int(b) for a, b in zip(A[m].tolist(), B[n].tolist()))


@pytest.mark.parametrize("qmax,K", [(127, 1024), (127, 6144), (7, 4096)])
def test_gemm_closed_form_all_qmax(qmax, K):
    A = np.full((2, K), qmax, np.int8)
    A[1] = -qmax
    B = np.full((3, K), qmax, np.int8)
    acc = oracle.gemm_s32(A, B)
    assert np.all(acc[0] == qmax * qmax * K) and np.all(acc[1] == -qmax * qmax * K)


def test_gemm_not_transposed():
    # acc[m, n] pairs row m of A with row n of B (both K-contiguous): a rank-one check.
    A = np.zeros((2, 128), np.int8)
    B = np.zeros((3, 128), np.int8)
    A[1, 7] = 3
    B[2, 7] = -5
    acc = oracle.gemm_s32(A, B)
    assert acc[1, 2] == -15 and np.count_nonzero(acc) == 1


def test_gemm_overflow_detected():
    A = np.full((1, 128 * 1100), 127, np.int8)
    with pytest.raises(OverflowError):
        oracle.gemm_s32(A, A)


def test_epilogue_golden_cases():
    for c in json.load(open(os.path.join(GOLD, "epilogue_cases.json")))["cases"]:
        acc = np.array([[c["acc"]]], np.int32)
        sx = np.array([c["s_x"]], np.float32)
        sw = np.array([c["s_w"]], np.float32)
        b = np.array([c["bias"]], np.float32)
        assert int(oracle.epilogue(acc, sx, sw, b, oracle.F16)[0, 0]) == c["f16"], c
        assert int(oracle.epilogue(acc, sx, sw, b, oracle.BF16)[0, 0]) == c["bf16"], c


def test_epilogue_zero_rows_and_columns_give_bias():
    rng = np.random.default_rng(1)
    acc = rng.integers(-10**6, 10**6, (4, 6)).astype(np.int32)
    acc[2, :] = 0      # zero X row
    acc[:, 3] = 0      # zero W row
    sx = rng.random(4).astype(np.float32)
    sw = rng.random(6).astype(np.float32)
    b = rng.normal(0, 0.01, 6).astype(np.float32)
    Y = oracle.epilogue(acc, sx, sw, b, oracle.F16)
    assert np.array_equal(Y[2], b.astype(np.float16).view(np.uint16))
    assert np.all(Y[:, 3] == b.astype(np.float16).view(np.uint16)[3])
    Yn = oracle.epilogue(acc, sx, sw, None, oracle.BF16)
    assert np.all(Yn[2] == 0)   # bias absent -> +0


@pytest.mark.parametrize("out_dtype", [oracle.F16, oracle.BF16])
def test_epilogue_matches_exact_fused_multiply_add(out_dtype):
    # v = RN32(f32(acc) * RN32(s_w * s_x) + bias) computed in exact rationals, then cast by the
    # library (numpy binary16 / torch bfloat16); the oracle must agree bit for bit.
    import torch
    rng = np.random.default_rng(7)
    M, N = 12, 10
    acc = rng.integers(-2**30, 2**30, (M, N)).astype(np.int32)
    acc[0, :] = rng.integers(-3000, 3000, N)
    sx = (rng.random(M) * 1e-2).astype(np.float32)
    sw = (rng.random(N) * 1e-3).astype(np.float32)
    b = rng.normal(0, 0.01, N).astype(np.float32)
    Y = oracle.epilogue(acc, sx, sw, b, out_dtype)
    for m in range(M):
        for n in range(N):
            af = np.float32(acc[m, n])                     # numpy int32 -> f32 is RNE
            sc = np.float32(sw[n]) * np.float32(sx[m])     # one binary32 product
            v = f32_nearest(Fraction(float(af)) * Fraction(float(sc)) + Fraction(float(b[n])))
            if out_dtype == oracle.F16:
                ref = int(np.array([v], np.float32).astype(np.float16).view(np.uint16)[0])
            else:
                ref = int(torch.tensor([float(v)], dtype=torch.float32).to(torch.bfloat16)
                          .view(torch.int16).item()) & 0xFFFF
            assert int(Y[m, n]) == ref, (m, n)
