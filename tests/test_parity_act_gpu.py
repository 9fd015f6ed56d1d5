"""GPU parity of the epilogue with a fused MLP activation (GELU, erf and tanh forms).

The accumulators stay bit-exact; the fp32 pre-activation is the plain epilogue's value; GELU is
evaluated in binary32 on the GPU and in binary64 by the oracle, so an output may be the adjacent
fp16/bf16 value only next to a rounding midpoint (tests.gpu_util.act_outputs_match), and such
elements must stay rare. Every GEMM kernel is covered: four waves per tile, eight waves
splitting K, 256 x 256 long-K tiles, Xq fragments in registers, weights resident in LDS,
row-major and tiled codes, int4 codes and the FP6 path. Every element is compared.
("SAM 3.1 Multiplex INT8/INT4 ConvRot" page, "Future improvements": fusion and fewer
dispatches; the activation itself is not on the pages.)
"""
import numpy as np
import pytest
import torch

import oracle
import w4a4_integer_quantized_amd as rq
from w4a4_integer_quantized_amd import synth
from tests.gpu_util import (IO_CODE, act_outputs_match, bits_from_dev, dev_from_bits, fp6_tile,
                            need_gpu, tile_codes)

pytestmark = pytest.mark.gpu

ACTS = [rq.RQ_ACT_GELU_ERF, rq.RQ_ACT_GELU_TANH]
assert (rq.RQ_ACT_GELU_ERF, rq.RQ_ACT_GELU_TANH) == (oracle.ACT_GELU_ERF, oracle.ACT_GELU_TANH)


def _codes(rng, rows, K, bits):
    q = 127 if bits == 8 else 7
    return rng.integers(-q, q + 1, (rows, K)).astype(np.int8)


def _scales(rng, M, N, K, bits):
    """Scales that put the pre-activation at a few units, where GELU bends."""
    q = 127 if bits == 8 else 7
    acc_sd = q * q / 3.0 * np.sqrt(K)
    sx = (0.5 + rng.random(M)).astype(np.float32) * np.float32(1.0 / np.sqrt(acc_sd))
    sw = (0.5 + rng.random(N)).astype(np.float32) * np.float32(2.0 / np.sqrt(acc_sd))
    b = rng.normal(0, 0.3, N).astype(np.float32)
    return sx, sw, b


# (M, N, K, bits, layout): launch shapes of every kernel that runs the epilogue.
CASES = [(300, 1040, 1024, 8, "tiled"),      # 4 waves per tile, ragged M and N
         (1000, 1040, 1024, 8, "tiled"),     # 36 tiles, 16 steps: 8 waves splitting K
         (4100, 2080, 3072, 8, "tiled"),     # > 256 tiles, K = 3072 bytes: 256 x 256 tiles
         (4100, 2064, 1536, 8, "tiled"),     # > 256 tiles, K = 1536 bytes: Xq in registers
         (4100, 3072, 1024, 8, "tiled"),     # N = 32 x 96, K = 1024: weights resident in LDS
         (600, 2064, 1024, 8, "rows"),       # row-major codes
         (2000, 6144, 3072, 4, "rows"),      # row-major int4 codes on enough tiles for the
                                             # 128-byte-row kernel without an activation
         (700, 1024, 2048, 4, "tiled"),      # int4 codes, split K
         (257, 512, 4096, 4, "fp6"),         # FP6 matrix cores, split K
         (600, 1040, 896, 4, "fp6")]         # FP6 matrix cores, 4 waves per tile


@pytest.mark.parametrize("M,N,K,bits,layout", CASES)
@pytest.mark.parametrize("act", ACTS)
def test_gemm_dequant_act_parity(M, N, K, bits, layout, act):
    need_gpu()
    print("act case act=%d M=%d N=%d K=%d bits=%d %s" % (act, M, N, K, bits, layout), flush=True)
    rng = np.random.default_rng(M + 7 * N + K + bits + 100 * act)
    A, B = _codes(rng, M, K, bits), _codes(rng, N, K, bits)
    sx, sw, b = _scales(rng, M, N, K, bits)
    if layout == "fp6":
        Ad = torch.from_numpy(fp6_tile(A, 256, pad_fill=0x3F)).cuda()
        Bd = torch.from_numpy(fp6_tile(B, 128, pad_fill=0x3F)).cuda()
        kw = dict(x_layout=rq.RQ_X_FP6, w_layout=rq.RQ_W_FP6)
    else:
        packed = oracle.pack_codes(A, bits)
        Ad = torch.from_numpy(tile_codes(packed, M, K, bits, pad_fill=0x77) if layout == "tiled" else packed).cuda()
        Bd = torch.from_numpy(oracle.pack_codes(B, bits)).cuda()
        kw = dict(x_layout=rq.RQ_X_TILED if layout == "tiled" else rq.RQ_X_ROWS)
    dev = lambda a: torch.from_numpy(a).cuda()
    rows = np.arange(M)
    ref_acc = oracle.gemm_s32(np.ascontiguousarray(A[rows]), B)
    for io in ("f16", "bf16"):
        Y = rq.gemm_dequant(Ad, dev(sx), Bd, dev(sw), dev(b), bits=bits, K=K, act=act,
                            out_dtype=torch.float16 if io == "f16" else torch.bfloat16, **kw)
        Y0 = rq.gemm_dequant(Ad, dev(sx), Bd, dev(sw), dev(b), bits=bits, K=K,
                             out_dtype=torch.float16 if io == "f16" else torch.bfloat16, **kw)
        torch.cuda.synchronize()
        ref, g64 = oracle.epilogue_act(ref_acc, sx[rows], sw, b, IO_CODE[io], act)
        v = oracle.epilogue_act(ref_acc, sx[rows], sw, b, IO_CODE[io], oracle.ACT_NONE)[1]
        ok, n, detail = act_outputs_match(bits_from_dev(Y)[rows], ref, g64, IO_CODE[io], v, act)
        assert ok, (io, detail)
        # the same launch without the activation is the plain epilogue, bit for bit
        assert np.array_equal(bits_from_dev(Y0)[rows], oracle.epilogue(ref_acc, sx[rows], sw, b, IO_CODE[io]))


@pytest.mark.parametrize("act", ACTS)
def test_gemm_dequant_act_wide_range(act):
    """Pre-activations from -12 to 40 (the negative tail down to binary32 values near 1e-32,
    the bend, the linear part) with no bias."""
    need_gpu()
    M, N, K = 256, 512, 128
    rng = np.random.default_rng(11 + act)
    A = np.zeros((M, K), np.int8)
    A[:, 0] = 1
    B = np.zeros((N, K), np.int8)
    B[:, 0] = 127
    sx = np.linspace(-12, 40, M).astype(np.float32) / np.float32(127.0)
    sw = (1.0 + rng.random(N) * 0.01).astype(np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    for io in ("f16", "bf16"):
        Y = rq.gemm_dequant(dev(A), dev(sx), dev(B), dev(sw), None, bits=8, act=act,
                            out_dtype=torch.float16 if io == "f16" else torch.bfloat16)
        torch.cuda.synchronize()
        acc = oracle.gemm_s32(A, B)
        ref, g64 = oracle.epilogue_act(acc, sx, sw, None, IO_CODE[io], act)
        v = oracle.epilogue_act(acc, sx, sw, None, IO_CODE[io], oracle.ACT_NONE)[1]
        ok, n, detail = act_outputs_match(bits_from_dev(Y), ref, g64, IO_CODE[io], v, act)
        assert ok, (io, detail)


@pytest.mark.parametrize("key,act,M", [("vit_mlp", rq.RQ_ACT_GELU_ERF, 300),
                                       ("dit", rq.RQ_ACT_GELU_TANH, 260)])
def test_rotq_linear_act_mlp_first_layer(key, act, M):
    """The first linear of an MLP pair with its GELU fused, from activations to output."""
    need_gpu()
    g = synth.generate(key, M=M, with_second_layer=False)
    cfg = g["cfg"]
    lin = cfg.linears[0] if key == "vit_mlp" else [l for l in cfg.linears if l.name == "w1"][0]
    W, b = g["W"][lin.name], g["bias"][lin.name]
    xb = g["x_bits"]
    Wq, ws = rq.quantize_weights(dev_from_bits(W, "f32"), bits=cfg.bits)
    Y = rq.rotq_linear(dev_from_bits(xb, cfg.io), Wq, ws, torch.from_numpy(b).cuda(), bits=cfg.bits, act=act)
    torch.cuda.synchronize()
    wc, _, wsr = oracle.quantize_weights(W, cfg.bits)
    ref = oracle.rotq_linear(xb, IO_CODE[cfg.io], wc, wsr, b, cfg.bits, act=act)
    ok, n, detail = act_outputs_match(bits_from_dev(Y), ref["Y"], ref["g64"], IO_CODE[cfg.io], ref["v"], act)
    assert ok, detail


def test_rotq_linear_act_full_size_sampled():
    """The ViT MLP pair at its full size (5184 tokens, 1024 -> 4096 -> 1024) with the erf GELU
    fused into fc1: fc1's output on sampled rows against the oracle, then fc2 on the GPU's own
    fc1 output, bit-exact against the oracle on sampled rows."""
    need_gpu()
    g = synth.generate("vit_mlp", with_second_layer=False)
    cfg = g["cfg"]
    fc1, fc2 = cfg.linears
    xb = g["x_bits"]
    Wq1, ws1 = rq.quantize_weights(dev_from_bits(g["W"]["fc1"], "f32"), bits=8)
    Wq2, ws2 = rq.quantize_weights(dev_from_bits(g["W"]["fc2"], "f32"), bits=8)
    b1, b2 = (torch.from_numpy(g["bias"][n]).cuda() for n in ("fc1", "fc2"))
    H = rq.rotq_linear(dev_from_bits(xb, cfg.io), Wq1, ws1, b1, bits=8, act=rq.RQ_ACT_GELU_ERF)
    Y = rq.rotq_linear(H, Wq2, ws2, b2, bits=8)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 1, 255, 256, cfg.M - 1, np.random.default_rng(9).choice(cfg.M, 40)])
    w1c, _, w1s = oracle.quantize_weights(g["W"]["fc1"], 8)
    ref1 = oracle.rotq_linear(np.ascontiguousarray(xb[rows]), IO_CODE[cfg.io], w1c, w1s, g["bias"]["fc1"], 8,
                              act=oracle.ACT_GELU_ERF)
    Hb = bits_from_dev(H)
    ok, n, detail = act_outputs_match(Hb[rows], ref1["Y"], ref1["g64"], IO_CODE[cfg.io], ref1["v"],
                                      oracle.ACT_GELU_ERF)
    assert ok, detail
    w2c, _, w2s = oracle.quantize_weights(g["W"]["fc2"], 8)
    ref2 = oracle.rotq_linear(np.ascontiguousarray(Hb[rows]), IO_CODE[cfg.io], w2c, w2s, g["bias"]["fc2"], 8)
    assert np.array_equal(bits_from_dev(Y)[rows], ref2["Y"])
