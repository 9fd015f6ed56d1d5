"""Pins for the oracle's MLP activation (GELU, erf and tanh forms) and its fused epilogue.

The pages leave the MLP activation unstated; the readings are the erf form for the ViT MLP and
the tanh form for the DiT MLP. These tests tie the oracle's binary64 GELU to things other than
itself: the normal CDF at 1, the odd-part identity GELU(x) - GELU(-x) = x, the asymptotes, an
independent implementation (torch's, in float64, where its 1 + erf / 1 + tanh form has no
cancellation), and the plain epilogue when the activation is off.
"""
import math

import numpy as np
import pytest
import torch

import oracle

ACTS = [(oracle.ACT_GELU_ERF, "none"), (oracle.ACT_GELU_TANH, "tanh")]


def test_gelu_erf_at_one_is_the_normal_cdf():
    # GELU(x) = x * Phi(x); Phi(1) = 0.8413447460685429... (standard normal table value)
    g = oracle.gelu_f64(np.array([1.0, 2.0, -1.0]), oracle.ACT_GELU_ERF)
    assert g[0] == pytest.approx(0.8413447460685429, rel=1e-15)
    assert g[1] == pytest.approx(2 * 0.9772498680518208, rel=1e-15)      # 2 * Phi(2)
    assert g[2] == pytest.approx(-(1 - 0.8413447460685429), rel=1e-14)   # -Phi(-1)


@pytest.mark.parametrize("act,_", ACTS)
def test_gelu_odd_part_identity(act, _):
    # Both forms are x * s(x) with s(x) + s(-x) = 1, so GELU(x) - GELU(-x) = x exactly in reals.
    x = np.linspace(-12, 12, 2401)
    d = oracle.gelu_f64(x, act) - oracle.gelu_f64(-x, act)
    assert np.max(np.abs(d - x) / np.maximum(np.abs(x), 1e-300)) < 1e-14


@pytest.mark.parametrize("act,_", ACTS)
def test_gelu_zero_and_asymptotes(act, _):
    g = oracle.gelu_f64(np.array([0.0, 30.0, 1e6, -30.0, -1e6]), act)
    assert g[0] == 0.0
    assert g[1] == 30.0 and g[2] == 1e6          # s(x) rounds to 1 in binary64
    assert -1e-100 < g[3] <= 0.0 and g[4] == 0.0  # s(x) vanishes (negative zero or underflow)


@pytest.mark.parametrize("act,approx", ACTS)
def test_gelu_matches_torch_float64(act, approx):
    # torch evaluates 0.5 x (1 + erf(x / sqrt 2)) / 0.5 x (1 + tanh(u)) in float64: an
    # independent implementation, accurate wherever 1 + erf (1 + tanh) does not cancel.
    x = np.linspace(-3, 10, 5201)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate=approx).numpy()
    g = oracle.gelu_f64(x, act)
    assert np.max(np.abs(g - ref) / np.maximum(np.abs(ref), 1e-300)) < 1e-12
    # And in absolute terms on the whole range (the tail values are tiny).
    x = np.linspace(-20, 20, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate=approx).numpy()
    assert np.max(np.abs(oracle.gelu_f64(x, act) - ref)) < 1e-14


def test_tanh_form_approximates_erf_form():
    # The tanh form is a published approximation of the erf form, within about 5e-4 absolute.
    x = np.linspace(-8, 8, 16001)
    d = oracle.gelu_f64(x, oracle.ACT_GELU_TANH) - oracle.gelu_f64(x, oracle.ACT_GELU_ERF)
    assert 1e-4 < np.max(np.abs(d)) < 1e-3


def test_gelu_tail_is_relatively_accurate():
    # For negative x the erfc form keeps full relative accuracy: x Phi(x) against the
    # continued-fraction tail Phi(x) ~ phi(x) / |x| * (1 - 1/x^2 + 3/x^4 - 15/x^6 + 105/x^8).
    x = np.array([-8.0, -10.0, -12.0])
    phi = np.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    tail = phi / np.abs(x) * (1 - 1 / x**2 + 3 / x**4 - 15 / x**6 + 105 / x**8 - 945 / x**10)
    g = oracle.gelu_f64(x, oracle.ACT_GELU_ERF)
    assert np.all(np.abs(g / (x * tail) - 1) < 2e-4)    # series truncation error, not cancellation


@pytest.mark.parametrize("out", [oracle.F16, oracle.BF16])
def test_epilogue_act_none_is_the_plain_epilogue(out):
    rng = np.random.default_rng(7)
    acc = rng.integers(-2**22, 2**22, (9, 32)).astype(np.int32)
    sx = (rng.random(9) * 1e-3).astype(np.float32)
    sw = (rng.random(32) * 1e-3).astype(np.float32)
    b = rng.normal(0, 0.1, 32).astype(np.float32)
    Y, g = oracle.epilogue_act(acc, sx, sw, b, out, oracle.ACT_NONE)
    assert np.array_equal(Y, oracle.epilogue(acc, sx, sw, b, out))
    v = g.astype(np.float32)
    assert np.array_equal(g, v.astype(np.float64))     # act 0 reports the fp32 value itself


@pytest.mark.parametrize("act,_", ACTS)
@pytest.mark.parametrize("out", [oracle.F16, oracle.BF16])
def test_epilogue_act_rounds_gelu_of_the_fp32_value(act, _, out):
    rng = np.random.default_rng(act * 10 + out)
    acc = rng.integers(-2**20, 2**20, (17, 48)).astype(np.int32)
    sx = (rng.random(17) * 4e-3).astype(np.float32)
    sw = (rng.random(48) * 4e-3).astype(np.float32)
    Y, g = oracle.epilogue_act(acc, sx, sw, None, out, act)
    # the pre-activation is the plain epilogue's fp32 value (no bias: +0)
    _, v = oracle.epilogue_act(acc, sx, sw, None, out, oracle.ACT_NONE)
    assert np.array_equal(g, oracle.gelu_f64(v, act))
    conv = oracle.f32_to_f16_bits if out == oracle.F16 else oracle.f32_to_bf16_bits
    assert np.array_equal(Y, conv(g.astype(np.float32)))
