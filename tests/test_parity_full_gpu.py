"""GPU parity at the workloads' full sizes, through the entry point and launch shapes that the
benchmark times (rq_rotq_linear with a caller-provided workspace), plus size edge cases.

Full size: every activation code and per-token scale (read back from the workspace, whose
layout is the tiled Xq then x_scale, each padded to 256 bytes) and every weight code and scale is
compared with the CPU oracle; the output Y is compared on a sample of rows (the first and
last rows, the rows around a 256-row tile edge, the ragged last tile and random rows) for
which the oracle runs the whole linear, all N columns. Properties that hold for every row
(max |code| = q_max on each nonzero row, codes within [-q_max, q_max]) are checked on all rows.
"""
import numpy as np
import pytest
import torch

import oracle
import w4a4_integer_quantized_amd as rq
from w4a4_integer_quantized_amd import synth
from tests.gpu_util import (IO_CODE, bits_from_dev, codes_np, compare_codes, dev_from_bits,
                            need_gpu, untile_codes, y_tolerance_ok)

pytestmark = pytest.mark.gpu


def _round256(n):
    return (n + 255) // 256 * 256


def _sample_rows(M, seed, n_random=48):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 127, 255, 256, 257, M - 1, M - 2, (M - 1) // 256 * 256, M // 2]
    rows = set(r for r in fixed if 0 <= r < M)
    rows.update(int(r) for r in rng.choice(M, min(M, n_random), replace=False))
    return np.array(sorted(rows), dtype=np.int64)


def _check_code_properties(codes, bits, K, scales):
    c = codes if bits == 8 else oracle.unpack_int4(codes, K)
    qmax = 127 if bits == 8 else 7
    amax = np.abs(c.astype(np.int32)).max(axis=1)
    assert amax.max(initial=0) <= qmax
    nz = scales != 0
    assert np.all(amax[nz] == qmax)
    assert np.all(amax[~nz] == 0)


@pytest.mark.parametrize("key", list(synth.CONFIGS))
def test_full_size_linear(key):
    need_gpu()
    g = synth.generate(key)
    cfg = g["cfg"]
    M, bits, io = cfg.M, cfg.bits, cfg.io
    rows = _sample_rows(M, cfg.seed + 100)
    print("full-size parity: %s M=%d bits=%d io=%s, %d sampled rows" % (cfg.workload, M, bits, io, len(rows)),
          flush=True)
    for lin in cfg.linears:
        xb = g["x_bits"] if lin.source == "x" else g["x2_bits"][lin.name]
        W, b = g["W"][lin.name], g["bias"][lin.name]
        K, N = lin.K, lin.N

        # Offline weights: all codes and scales.
        Wq, ws = rq.quantize_weights(dev_from_bits(W, "f32"), bits=bits)
        wc, _, wsr = oracle.quantize_weights(W, bits)
        torch.cuda.synchronize()
        wref_c, wref_s, wref_p = oracle.quantize_rows(W, oracle.F32, bits, want_pre=True)
        assert compare_codes(codes_np(Wq), wref_c, wref_p, bits, K) == 0, lin.name
        assert np.array_equal(ws.cpu().numpy().view(np.uint32), wsr.view(np.uint32)), lin.name

        # The timed entry point with an explicit workspace.
        X = dev_from_bits(xb, io)
        bd = torch.from_numpy(b).cuda()
        need = rq.workspace_size(M, K, bits)
        wsbuf = torch.empty((need,), dtype=torch.uint8, device="cuda")
        Y = rq.rotq_linear(X, Wq, ws, bd, bits=bits, workspace=wsbuf)
        torch.cuda.synchronize()

        # Every activation code and scale (the workspace holds the codes in the tiled layout).
        cb = rq.rq_codes_bytes(M, K, rq.make_cfg(bits, x_layout=rq.RQ_X_TILED))
        xs = wsbuf[_round256(cb):_round256(cb) + 4 * M].view(torch.float32)
        xq_np = untile_codes(wsbuf[:cb].cpu().numpy(), M, K, bits)
        xs_np = xs.cpu().numpy()
        ref_c, ref_s, ref_p = oracle.quantize_rows(xb, IO_CODE[io], bits, want_pre=True)
        nmis = compare_codes(xq_np, ref_c, ref_p, bits, K)
        assert np.array_equal(xs_np.view(np.uint32), ref_s.view(np.uint32)), lin.name
        _check_code_properties(xq_np, bits, K, xs_np)
        del ref_p

        # Sampled rows of Y: the oracle's whole linear on those tokens.
        ref = oracle.rotq_linear(np.ascontiguousarray(xb[rows]), IO_CODE[io], wc, wsr, b, bits)
        got = bits_from_dev(Y[torch.from_numpy(rows).cuda()])
        ok, maxerr = y_tolerance_ok(got, ref["Y"], io)
        assert ok, (lin.name, maxerr)
        if nmis == 0:
            assert np.array_equal(got, ref["Y"]), lin.name
        print("  %s: K=%d N=%d codes %d mismatches, Y rows bit-exact=%s" %
              (lin.name, K, N, nmis, bool(np.array_equal(got, ref["Y"]))), flush=True)
        del X, Y, wsbuf, xs
        torch.cuda.empty_cache()


def test_empty_inputs_are_no_ops():
    need_gpu()
    for bits in (8, 4):
        X = torch.empty((0, 1024), dtype=torch.float16, device="cuda")
        Xq, xs = rq.rotate_quantize(X, bits=bits)
        assert Xq.shape[0] == 0 and xs.shape[0] == 0
        Wq, ws = rq.quantize_weights(torch.randn(64, 1024, device="cuda"), bits=bits)
        Y = rq.rotq_linear(X, Wq, ws, bits=bits)
        assert Y.shape == (0, 64)
        Yd = rq.gemm_dequant(Xq, xs, Wq, ws, bits=bits, K=1024)
        assert Yd.shape == (0, 64)
        acc = rq.gemm_s32(Xq, Wq, bits=bits, K=1024)
        assert acc.shape == (0, 64)
    # An empty weight matrix quantizes to nothing.
    Wq, ws = rq.quantize_weights(torch.empty((0, 256), device="cuda"))
    torch.cuda.synchronize()
    assert Wq.shape == (0, 256) and ws.shape == (0,)


@pytest.mark.parametrize("bits", [8, 4])
def test_maximum_k(bits):
    """K = 131072, the largest supported reduction: the generic two-pass rotate kernel and the
    GEMM's longest k loop, plus the accumulator bound q_max^2 * K reached exactly."""
    need_gpu()
    K, M, N = 131072, 5, 32
    rng = np.random.default_rng(77 + bits)
    x = synth.random_rows(rng, M, K, "normal", 20, 40.0)
    W = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    b = rng.normal(0, 0.01, N).astype(np.float32)
    xb = synth.to_io_bits(x, "f16")
    Wq, ws = rq.quantize_weights(dev_from_bits(W, "f32"), bits=bits)
    Y = rq.rotq_linear(dev_from_bits(xb, "f16"), Wq, ws, torch.from_numpy(b).cuda(), bits=bits)
    torch.cuda.synchronize()
    wc, _, wsr = oracle.quantize_weights(W, bits)
    ref = oracle.rotq_linear(xb, oracle.F16, wc, wsr, b, bits)
    assert np.array_equal(bits_from_dev(Y), ref["Y"])

    # All codes at +q_max against all at -q_max (and +q_max): acc = -/+ q_max^2 K, the extreme
    # the int32 accumulator has to hold.
    q = 127 if bits == 8 else 7
    codes_x = np.full((3, K), q, np.int8)
    codes_x[1] = -q
    codes_w = np.full((16, K), q, np.int8)
    codes_w[1::2] = -q
    to_dev = (lambda c: torch.from_numpy(c).cuda()) if bits == 8 else \
        (lambda c: torch.from_numpy(oracle.pack_int4(c)).cuda())
    acc = rq.gemm_s32(to_dev(codes_x), to_dev(codes_w), bits=bits, K=K).cpu().numpy()
    sign = np.where(np.arange(16) % 2 == 0, 1, -1)
    expect = np.stack([sign, -sign, sign]) * (q * q * K)
    assert np.array_equal(acc, expect)
