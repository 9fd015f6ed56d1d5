"""GPU parity of the weight quantizer's alternative scale rules against the CPU oracle.

RQ_W_MSE: per-row MSE-optimized clipping ('SAM 3.1 Multiplex INT8/INT4 ConvRot' page,
'Quantization recipe', step 3). Both sides evaluate every candidate's binary64 error in the
same order, so the chosen clip, the codes and the scales must agree bit for bit.
RQ_W_TENSOR: one tensor-wise scale (the HSWQ ConvRot model card's int8_tensorwise).
The linear run on such weights is checked end to end as well (the GEMM only sees w_scale).
"""
import numpy as np
import pytest
import torch

import oracle
import w4a4_integer_quantized_amd as rq
from w4a4_integer_quantized_amd import synth
from tests.gpu_util import IO_CODE, bits_from_dev, codes_np, dev_from_bits, need_gpu

pytestmark = pytest.mark.gpu


def _weights(rng, N, K, kind):
    if kind == "normal":
        return rng.normal(0.0, 0.02, (N, K)).astype(np.float32)
    if kind == "laplace":
        return rng.laplace(0.0, 0.02, (N, K)).astype(np.float32)
    # Rows of several shapes: outlier channels, a zero row, a constant-magnitude rotated row,
    # a row of tiny values.
    W = rng.normal(0.0, 0.02, (N, K)).astype(np.float32)
    W[:, rng.choice(K, 4, replace=False)] *= 40
    W[1] = 0
    W[2] = 0
    W[2, 0] = 0.5                     # rotates to +-0.5 over the first block, 0 elsewhere
    W[3] *= np.float32(1e-20)
    return W


def _to_io(W, io):
    return W if io == "f32" else synth.to_io_bits(W, io)


def _expected(Wio, io, bits, mode):
    if mode == rq.RQ_W_MSE:
        c, s, idx, _ = oracle.quantize_rows_mse(Wio, IO_CODE[io], bits)
    else:
        c, s, _ = oracle.quantize_tensorwise(Wio, IO_CODE[io], bits)
        idx = None
    return (c if bits == 8 else oracle.pack_int4(c)), s, idx


CASES = [  # (N, K, bits, io, kind)
    (64, 128, 4, "f32", "mixed"),
    (48, 384, 8, "f16", "mixed"),
    (80, 1024, 4, "bf16", "laplace"),
    (37, 4096, 4, "f32", "normal"),
    (16, 1536, 8, "bf16", "mixed"),
    (5, 131072, 4, "f16", "mixed"),
]


@pytest.mark.parametrize("mode", [rq.RQ_W_MSE, rq.RQ_W_TENSOR])
@pytest.mark.parametrize("N,K,bits,io,kind", CASES)
def test_weight_mode_parity(mode, N, K, bits, io, kind):
    need_gpu()
    print("weight mode %d: N=%d K=%d bits=%d io=%s %s" % (mode, N, K, bits, io, kind), flush=True)
    rng = np.random.default_rng(N * 7 + K + bits)
    Wio = _to_io(_weights(rng, N, K, kind), io)
    Wq, ws = rq.quantize_weights(dev_from_bits(Wio, io), bits=bits, w_scale_mode=mode)
    torch.cuda.synchronize()
    c_ref, s_ref, idx = _expected(Wio, io, bits, mode)
    assert np.array_equal(ws.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(codes_np(Wq), c_ref)
    if mode == rq.RQ_W_MSE and bits == 4 and kind != "mixed":
        assert (idx > 0).mean() > 0.9     # 4-bit bell-shaped rows clip


@pytest.mark.parametrize("mode", [rq.RQ_W_MSE, rq.RQ_W_TENSOR])
@pytest.mark.parametrize("key", ["vit_mlp", "w4a4"])
def test_weight_mode_full_size_and_linear(mode, key):
    """A workload's full weight matrices, then the fused linear on such weights for a sample of
    tokens (the oracle runs the same linear from its own weight codes)."""
    need_gpu()
    g = synth.generate(key, M=300, with_second_layer=False)
    cfg = g["cfg"]
    lin = cfg.linears[0]
    W, b = g["W"][lin.name], g["bias"][lin.name]
    print("weight mode %d full size: %s %s N=%d K=%d bits=%d" % (mode, key, lin.name, lin.N, lin.K, cfg.bits),
          flush=True)
    Wq, ws = rq.quantize_weights(dev_from_bits(W, "f32"), bits=cfg.bits, w_scale_mode=mode)
    torch.cuda.synchronize()
    c_ref, s_ref, _ = _expected(W, "f32", cfg.bits, mode)
    assert np.array_equal(ws.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(codes_np(Wq), c_ref)
    if mode == rq.RQ_W_TENSOR:
        assert np.all(s_ref == s_ref[0])

    xb = g["x_bits"]
    Y = rq.rotq_linear(dev_from_bits(xb, cfg.io), Wq, ws, torch.from_numpy(b).cuda(), bits=cfg.bits)
    torch.cuda.synchronize()
    wc = c_ref if cfg.bits == 8 else oracle.unpack_int4(c_ref, lin.K)
    ref = oracle.rotq_linear(xb, IO_CODE[cfg.io], wc, s_ref, b, cfg.bits)
    assert np.array_equal(bits_from_dev(Y), ref["Y"])


def test_weight_modes_zero_matrix():
    need_gpu()
    for mode in (rq.RQ_W_MSE, rq.RQ_W_TENSOR):
        for bits in (8, 4):
            Wq, ws = rq.quantize_weights(torch.zeros((32, 256), device="cuda"), bits=bits, w_scale_mode=mode)
            torch.cuda.synchronize()
            assert not Wq.cpu().numpy().any() and not ws.cpu().numpy().any()


def test_mixed_int8_int4_mlp_pair():
    """Mixed precision per layer ('SAM 3.1 Multiplex INT8/INT4 ConvRot', 'Why these two
    variants': a mixed INT4/INT8 checkpoint): fc1 as W8A8 and fc2 as W4A4 through the same
    entry points, each checked against the oracle on all rows."""
    need_gpu()
    g = synth.generate("vit_mlp", M=260)
    cfg = g["cfg"]
    for lin, bits in zip(cfg.linears, (8, 4)):
        xb = g["x_bits"] if lin.source == "x" else g["x2_bits"][lin.name]
        W, b = g["W"][lin.name], g["bias"][lin.name]
        Wq, ws = rq.quantize_weights(dev_from_bits(W, "f32"), bits=bits)
        Y = rq.rotq_linear(dev_from_bits(xb, cfg.io), Wq, ws, torch.from_numpy(b).cuda(), bits=bits)
        torch.cuda.synchronize()
        wc, _, wsr = oracle.quantize_weights(W, bits)
        ref = oracle.rotq_linear(xb, IO_CODE[cfg.io], wc, wsr, b, bits)
        assert np.array_equal(bits_from_dev(Y), ref["Y"]), (lin.name, bits)
