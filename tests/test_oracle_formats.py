"""Pins for the oracle's number-format conversions.

The epilogue stores fp16 / bf16 with round-to-nearest-even; the oracle implements both casts
by hand from the format definitions, so they are checked here against library casts
(numpy's binary16, torch's bfloat16) over every input class that matters.
"""
import numpy as np
import pytest
import torch

import oracle


def _interesting_f32(n=200000, seed=0):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    extra = np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 65536.0, -65520.0,
                      6.1035156e-05, 5.9604645e-08, 2.9802322e-08, 2.98023259e-08, 1e-9,
                      1.0 + 2**-11, 1.0 + 3 * 2**-11, 2049.0, 2051.0, 3.4e38, -3.4e38,
                      1.0 + 2**-8, 1.0 + 3 * 2**-8, np.inf, -np.inf], np.float32)
    # values near f16 rounding boundaries: k * 2^-11 around 1, and subnormal ties
    k = np.arange(-3000, 3000, dtype=np.float64)
    ties = np.concatenate([1.0 + k * 2.0**-12, k * 2.0**-25, 1024 + k * 2.0**-1]).astype(np.float32)
    return np.concatenate([vals, extra, ties])


def test_f32_to_f16_matches_numpy():
    x = _interesting_f32()
    x = x[~np.isnan(x)]
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.f32_to_f16_bits(x)
    assert np.array_equal(got, ref)


def test_f32_to_f16_nan_stays_nan():
    got = oracle.f32_to_f16_bits(np.array([np.nan, -np.nan], np.float32))
    assert np.all(np.isnan(got.view(np.float16)))


def test_f16_to_f32_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    got = oracle.f16_bits_to_f32(h)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_bf16_matches_torch():
    x = _interesting_f32(seed=1)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16_bits(x)
    assert np.array_equal(got, ref)


def test_bf16_to_f32_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    got = oracle.bf16_bits_to_f32(h)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("v,f16,bf16", [(1.0 + 2**-11, 0x3C00, None), (1.0 + 3 * 2**-11, 0x3C02, None),
                                        (1.0 + 2**-8, None, 0x3F80), (1.0 + 3 * 2**-8, None, 0x3F82),
                                        (65520.0, 0x7C00, None), (126.0, 0x57E0, 0x42FC)])
def test_round_half_even_hand_cases(v, f16, bf16):
    # Exactly halfway cases go to the even neighbour; 65520 is half an ulp above 65504 -> inf.
    x = np.array([v], np.float32)
    if f16 is not None:
        assert int(oracle.f32_to_f16_bits(x)[0]) == f16
    if bf16 is not None:
        assert int(oracle.f32_to_bf16_bits(x)[0]) == bf16
