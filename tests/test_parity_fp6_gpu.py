"""GPU parity of the W4A4 path on the FP6 matrix cores (4-bit codes stored as FP6 E2M3 tiles).

Every code in [-7, 7] is exactly an FP6 E2M3 value and the products and sums stay exact
integers in fp32, so this path must reproduce the oracle bit for bit: the same codes and scales
(decoded from the FP6 tiles), the same int32 accumulators and the same fp16/bf16 outputs.
('SAM 3.1 Multiplex INT8/INT4 ConvRot' page, 'Downloads' and 'Quantization recipe': W4A4
operations, INT4 multiplication where the hardware has it.)
"""
import numpy as np
import pytest
import torch

import oracle
import w4a4_integer_quantized_amd as rq
from w4a4_integer_quantized_amd import synth
from tests.gpu_util import (IO_CODE, bits_from_dev, compare_codes, dev_from_bits, fp6_tile,
                            fp6_untile, need_gpu)

pytestmark = pytest.mark.gpu

FP6X = rq.make_cfg(4, x_layout=rq.RQ_X_FP6)
FP6W = rq.make_cfg(4, w_layout=rq.RQ_W_FP6)


def _rows(seed, M, K, io, zero_rows=()):
    rng = np.random.default_rng(seed)
    x = synth.random_rows(rng, M, K, "laplace", max(1, K // 100), 30.0)
    for r in zero_rows:
        x[r] = 0
    return (x if io == "f32" else synth.to_io_bits(x, io)), x


@pytest.mark.parametrize("K,M", [(128, 1), (256, 37), (384, 33), (512, 529), (640, 9), (1024, 300),
                                 (1536, 129), (2176, 11), (3072, 13), (4096, 257), (6144, 19),
                                 (16384, 3)])
@pytest.mark.parametrize("io", ["f16", "bf16", "f32"])
def test_rotate_quantize_fp6_tiles(K, M, io):
    """Activation codes as FP6 tiles decode to exactly the oracle's 4-bit codes: the quad kernel,
    which writes FP6 tiles, at every slot shape it takes (K = 128 .. 16384, ragged M over several
    256-row panels) and the generic kernel (K = 2176)."""
    need_gpu()
    xb, _ = _rows(K + M, M, K, io, zero_rows=(0,) if M > 1 else ())
    Xt, xs = rq.rotate_quantize(dev_from_bits(xb, io), bits=4, x_layout=rq.RQ_X_FP6)
    torch.cuda.synchronize()
    assert Xt.numel() == rq.rq_codes_bytes(M, K, FP6X)
    got = fp6_untile(Xt.cpu().numpy(), M, K, 256)
    ref_c, ref_s, ref_p = oracle.quantize_rows(xb, IO_CODE[io], 4, want_pre=True)
    compare_codes(oracle.pack_int4(got), ref_c, ref_p, 4, K)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


@pytest.mark.parametrize("mode", [rq.RQ_W_ABSMAX, rq.RQ_W_MSE, rq.RQ_W_TENSOR])
@pytest.mark.parametrize("N,K", [(16, 128), (100, 384), (1024, 4096), (48, 2176), (300, 1024),
                                 (130, 640)])
def test_quantize_weights_fp6_tiles(mode, N, K):
    need_gpu()
    rng = np.random.default_rng(N + K + mode)
    W = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    W[:, rng.choice(K, 3, replace=False)] *= 30
    Wt, ws = rq.quantize_weights(dev_from_bits(W, "f32"), bits=4, w_scale_mode=mode, w_layout=rq.RQ_W_FP6)
    torch.cuda.synchronize()
    assert Wt.numel() == rq.rq_weight_bytes(N, K, FP6W)
    got = fp6_untile(Wt.cpu().numpy(), N, K, 128)
    if mode == rq.RQ_W_ABSMAX:
        ref_c, ref_s, _ = oracle.quantize_rows(W, oracle.F32, 4)
    elif mode == rq.RQ_W_MSE:
        ref_c, ref_s, _, _ = oracle.quantize_rows_mse(W, oracle.F32, 4)
    else:
        ref_c, ref_s, _ = oracle.quantize_tensorwise(W, oracle.F32, 4)
    assert np.array_equal(got, ref_c)
    assert np.array_equal(ws.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


def _codes(rng, rows, K):
    c = rng.integers(-7, 8, (rows, K)).astype(np.int8)
    c[rng.random(rows) < 0.05] = 7          # a few all-q_max rows: extreme accumulators
    return c


# Both launch shapes of the FP6 kernel (one or two wave groups per tile), ragged M and N, K from
# one 128-block to 8192.
FP6_GEMM_CASES = [(1, 16, 128), (37, 48, 256), (255, 272, 1024), (257, 256, 384), (600, 1040, 1024),
                  (300, 512, 4096), (129, 64, 8192), (1000, 1040, 896), (4096, 2064, 1024),
                  (5184, 1024, 4096)]


@pytest.mark.parametrize("M,N,K", FP6_GEMM_CASES)
def test_gemm_fp6_parity(M, N, K):
    need_gpu()
    print("fp6 gemm M=%d N=%d K=%d" % (M, N, K), flush=True)
    rng = np.random.default_rng(M * 3 + N + K)
    A, B = _codes(rng, M, K), _codes(rng, N, K)
    At = torch.from_numpy(fp6_tile(A, 256, pad_fill=0x3F)).cuda()
    Bt = torch.from_numpy(fp6_tile(B, 128, pad_fill=0x3F)).cuda()
    sx = (rng.random(M) * 0.05).astype(np.float32)
    sw = (rng.random(N) * 2e-4).astype(np.float32)
    b = rng.normal(0, 0.01, N).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).cuda()
    acc = rq.gemm_s32(At, Bt, bits=4, K=K, M=M, N=N, x_layout=rq.RQ_X_FP6, w_layout=rq.RQ_W_FP6)
    Y = rq.gemm_dequant(At, dev(sx), Bt, dev(sw), dev(b), bits=4, K=K, x_layout=rq.RQ_X_FP6,
                        w_layout=rq.RQ_W_FP6, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.arange(M) if M * N * K < 2e9 else np.unique(np.r_[np.arange(64), np.arange(M - 64, M),
                                                               np.random.default_rng(1).choice(M, 64)])
    ref_acc = oracle.gemm_s32(np.ascontiguousarray(A[rows]), B)
    assert np.array_equal(acc.cpu().numpy()[rows], ref_acc)
    assert np.array_equal(bits_from_dev(Y)[rows], oracle.epilogue(ref_acc, sx[rows], sw, b, oracle.BF16))


def test_gemm_fp6_extreme_accumulators():
    """K = 131072 with every code at +-7: acc = +-49 K = +-6422528, exact in fp32 (< 2^24)."""
    need_gpu()
    K = 131072
    A = np.full((3, K), 7, np.int8)
    A[1] = -7
    B = np.full((16, K), 7, np.int8)
    B[1::2] = -7
    acc = rq.gemm_s32(torch.from_numpy(fp6_tile(A, 256)).cuda(), torch.from_numpy(fp6_tile(B, 128)).cuda(),
                      bits=4, K=K, M=3, N=16, x_layout=rq.RQ_X_FP6, w_layout=rq.RQ_W_FP6).cpu().numpy()
    sign = np.where(np.arange(16) % 2 == 0, 1, -1)
    assert np.array_equal(acc, np.stack([sign, -sign, sign]) * (49 * K))


@pytest.mark.parametrize("M,N,K,io", [(1, 16, 128, "f16"), (300, 1040, 1024, "bf16"), (257, 512, 4096, "f16"),
                                      (70, 256, 2176, "bf16")])
def test_rotq_linear_fp6_small(M, N, K, io):
    need_gpu()
    xb, _ = _rows(M + N + K, M, K, io, zero_rows=(0,) if M > 1 else ())
    rng = np.random.default_rng(K)
    W = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    b = rng.normal(0, 0.01, N).astype(np.float32)
    Wt, ws = rq.quantize_weights(dev_from_bits(W, "f32"), bits=4, w_layout=rq.RQ_W_FP6)
    Y = rq.rotq_linear(dev_from_bits(xb, io), Wt, ws, torch.from_numpy(b).cuda(), bits=4,
                       w_layout=rq.RQ_W_FP6)
    torch.cuda.synchronize()
    wc, _, wsr = oracle.quantize_weights(W, 4)
    ref = oracle.rotq_linear(xb, IO_CODE[io], wc, wsr, b, 4)
    assert np.array_equal(bits_from_dev(Y), ref["Y"])


def test_rotq_linear_fp6_full_size():
    """The W4A4 workload (5184 tokens, K = 4096, N = 1024) on the FP6 path: every activation code
    and scale from the workspace, and the output on sampled rows, against the oracle; and the
    same output as the int8-MFMA path bit for bit."""
    need_gpu()
    g = synth.generate("w4a4", with_second_layer=False)
    cfg = g["cfg"]
    lin = cfg.linears[0]
    M, K, N = cfg.M, lin.K, lin.N
    W, b = g["W"][lin.name], g["bias"][lin.name]
    xb = g["x_bits"]
    Wt, ws = rq.quantize_weights(dev_from_bits(W, "f32"), bits=4, w_layout=rq.RQ_W_FP6)
    Wr, ws_r = rq.quantize_weights(dev_from_bits(W, "f32"), bits=4)
    X = dev_from_bits(xb, cfg.io)
    bd = torch.from_numpy(b).cuda()
    need = rq.workspace_size(M, K, 4, w_layout=rq.RQ_W_FP6)
    wsbuf = torch.empty((need,), dtype=torch.uint8, device="cuda")
    Y = rq.rotq_linear(X, Wt, ws, bd, bits=4, workspace=wsbuf, w_layout=rq.RQ_W_FP6)
    Yr = rq.rotq_linear(X, Wr, ws_r, bd, bits=4)
    torch.cuda.synchronize()
    assert torch.equal(ws, ws_r)
    assert torch.equal(Y, Yr)
    cb = rq.rq_codes_bytes(M, K, FP6X)
    xq = fp6_untile(wsbuf[:cb].cpu().numpy(), M, K, 256)
    xs = wsbuf[(cb + 255) // 256 * 256:(cb + 255) // 256 * 256 + 4 * M].view(torch.float32).cpu().numpy()
    ref_c, ref_s, ref_p = oracle.quantize_rows(xb, IO_CODE[cfg.io], 4, want_pre=True)
    compare_codes(oracle.pack_int4(xq), ref_c, ref_p, 4, K)
    assert np.array_equal(xs.view(np.uint32), ref_s.view(np.uint32))
    rows = np.unique(np.r_[0, 1, 255, 256, M - 1, np.random.default_rng(5).choice(M, 40)])
    wc, _, wsr = oracle.quantize_weights(W, 4)
    ref = oracle.rotq_linear(np.ascontiguousarray(xb[rows]), IO_CODE[cfg.io], wc, wsr, b, 4)
    assert np.array_equal(bits_from_dev(Y[torch.from_numpy(rows).cuda()]), ref["Y"])
