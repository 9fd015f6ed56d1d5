"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Bar: codes, scales and int32 accumulators bit-exact (a code may differ only if its
pre-rounding value lies within one fp32 ulp of a .5 boundary, at most 1e-5 of codes);
fp16 / bf16 outputs within max|err| <= 1e-3 + 2^-9 |ref| -- and, because the kernels follow
the same fp32 operation order as the oracle, bit-identical as well.
"""
import numpy as np
import pytest
import torch

import oracle
import w4a4_integer_quantized_amd as rq
from w4a4_integer_quantized_amd import synth
from tests.gpu_util import (IO_CODE, bits_from_dev, codes_np, compare_codes, dev_from_bits,
                            need_gpu, tile_codes, untile_codes, y_tolerance_ok)

pytestmark = pytest.mark.gpu


def _rows(seed, M, K, io, zero_rows=(), dist="normal"):
    rng = np.random.default_rng(seed)
    x = synth.random_rows(rng, M, K, dist, max(1, K // 100), 40.0)
    for r in zero_rows:
        if r < M:
            x[r] = 0
    if io == "f32":
        return x, x
    return synth.to_io_bits(x, io), None


# (K, M) pairs cover every kernel shape. Coalesced kernel (nb = K / 128 = G * NI): G = 1 with
# NI = 1..4 (K = 128 .. 512), G = 2 (768, 1024), G = 4 (1536, 2048), G = 12 (3072, 4608; three
# waves per row), G = 16 (4096, 6144, 8192; four waves per row); the quad kernel (K = 640:
# 5 blocks, K = 16384: four waves per row); the generic two-pass kernel (K = 2176, 17 blocks).
# M spans ragged tails.
RQ_CASES = [(128, 1), (128, 37), (256, 5), (384, 33), (512, 23), (640, 9), (768, 17),
            (1024, 300), (1536, 129), (2048, 41), (2176, 11), (3072, 13), (4096, 70), (4608, 5),
            (6144, 19), (8192, 6), (16384, 3)]


@pytest.mark.parametrize("K,M", RQ_CASES)
@pytest.mark.parametrize("io,bits", [("f16", 8), ("bf16", 8), ("f16", 4), ("f32", 8), ("f32", 4)])
def test_rotate_quantize_parity(K, M, io, bits):
    need_gpu()
    xb, _ = _rows(K + M + bits, M, K, io, zero_rows=(0, M - 1) if M > 2 else ())
    Xd = dev_from_bits(xb, io)
    Xq, xs = rq.rotate_quantize(Xd, bits=bits)
    torch.cuda.synchronize()
    ref_c, ref_s, ref_p = oracle.quantize_rows(xb, IO_CODE[io], bits, want_pre=True)
    compare_codes(codes_np(Xq), ref_c, ref_p, bits, K)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


@pytest.mark.parametrize("K,M", [(128, 1), (128, 529), (384, 33), (640, 9), (1024, 300),
                                 (1536, 257), (2176, 11), (3072, 13), (4096, 70), (6144, 19)])
@pytest.mark.parametrize("io,bits", [("f16", 8), ("bf16", 8), ("f16", 4)])
def test_rotate_quantize_tiled_layout(K, M, io, bits):
    """The tiled activation-code layout holds exactly the row-major codes (and the oracle's)."""
    need_gpu()
    xb, _ = _rows(K + M + bits + 7, M, K, io, zero_rows=(0,) if M > 1 else ())
    Xd = dev_from_bits(xb, io)
    Xt, st = rq.rotate_quantize(Xd, bits=bits, x_layout=rq.RQ_X_TILED)
    Xr, sr = rq.rotate_quantize(Xd, bits=bits)
    torch.cuda.synchronize()
    assert Xt.numel() == rq.rq_codes_bytes(M, K, rq.make_cfg(bits, x_layout=rq.RQ_X_TILED))
    got = untile_codes(Xt.cpu().numpy(), M, K, bits)
    assert np.array_equal(got.view(np.uint8), codes_np(Xr).view(np.uint8))
    assert torch.equal(st, sr)
    ref_c, ref_s, ref_p = oracle.quantize_rows(xb, IO_CODE[io], bits, want_pre=True)
    compare_codes(got, ref_c, ref_p, bits, K)
    assert np.array_equal(st.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


@pytest.mark.parametrize("key", list(synth.CONFIGS))
def test_quantize_weights_parity(key):
    need_gpu()
    g = synth.generate(key, M=8, with_second_layer=False)
    bits = g["cfg"].bits
    for name, W in g["W"].items():
        Wq, ws = rq.quantize_weights(dev_from_bits(W, "f32"), bits=bits)
        torch.cuda.synchronize()
        ref_c, ref_s, ref_p = oracle.quantize_rows(W, oracle.F32, bits, want_pre=True)
        assert compare_codes(codes_np(Wq), ref_c, ref_p, bits, W.shape[1]) == 0, name
        assert np.array_equal(ws.cpu().numpy().view(np.uint32), ref_s.view(np.uint32)), name


GEMM_CASES = [(1, 16, 128, 8), (37, 48, 256, 8), (255, 272, 1024, 8), (257, 256, 384, 8),
              (600, 1040, 1024, 8), (300, 512, 4096, 8), (129, 64, 6144, 8),
              (1, 16, 128, 4), (1, 16, 256, 4), (77, 48, 384, 4), (200, 272, 1024, 4),
              (517, 1024, 4096, 4)]


def _random_codes(rng, rows, K, bits):
    q = 127 if bits == 8 else 7
    c = rng.integers(-q, q + 1, (rows, K)).astype(np.int8)
    c[rng.random(rows) < 0.05] = q           # a few all-q_max rows: extreme accumulators
    return c


@pytest.mark.parametrize("M,N,K,bits", GEMM_CASES)
def test_gemm_s32_parity(M, N, K, bits):
    need_gpu()
    rng = np.random.default_rng(M * N + K)
    A = _random_codes(rng, M, K, bits)
    B = _random_codes(rng, N, K, bits)
    Ad = torch.from_numpy(oracle.pack_codes(A, bits)).cuda()
    Bd = torch.from_numpy(oracle.pack_codes(B, bits)).cuda()
    acc = rq.gemm_s32(Ad, Bd, bits=bits, K=K)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), oracle.gemm_s32(A, B))


@pytest.mark.parametrize("M,N,K,bits", GEMM_CASES)
def test_gemm_tiled_layout_parity(M, N, K, bits):
    """GEMM on tiled activation codes (pad rows filled with garbage, which must not matter)."""
    need_gpu()
    rng = np.random.default_rng(M * N + K + 17)
    A = _random_codes(rng, M, K, bits)
    B = _random_codes(rng, N, K, bits)
    At = torch.from_numpy(tile_codes(oracle.pack_codes(A, bits), M, K, bits, pad_fill=0x77)).cuda()
    Bd = torch.from_numpy(oracle.pack_codes(B, bits)).cuda()
    acc = rq.gemm_s32(At, Bd, bits=bits, K=K, x_layout=rq.RQ_X_TILED, M=M)
    sx = (rng.random(M) * 0.05).astype(np.float32)
    sw = (rng.random(N) * 2e-4).astype(np.float32)
    b = rng.normal(0, 0.01, N).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).cuda()
    Y = rq.gemm_dequant(At, dev(sx), Bd, dev(sw), dev(b), bits=bits, K=K, x_layout=rq.RQ_X_TILED)
    torch.cuda.synchronize()
    ref_acc = oracle.gemm_s32(A, B)
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    assert np.array_equal(bits_from_dev(Y), oracle.epilogue(ref_acc, sx, sw, b, oracle.F16))


@pytest.mark.parametrize("M,N,K,bits", GEMM_CASES[::2])
@pytest.mark.parametrize("io", ["f16", "bf16"])
@pytest.mark.parametrize("with_bias", [True, False])
def test_gemm_dequant_parity(M, N, K, bits, io, with_bias):
    need_gpu()
    rng = np.random.default_rng(M + N + K + bits)
    A = _random_codes(rng, M, K, bits)
    B = _random_codes(rng, N, K, bits)
    sx = (rng.random(M) * 0.05).astype(np.float32)
    sw = (rng.random(N) * 2e-4).astype(np.float32)
    b = rng.normal(0, 0.01, N).astype(np.float32) if with_bias else None
    dev = lambda a: torch.from_numpy(a).cuda()
    Y = rq.gemm_dequant(dev(oracle.pack_codes(A, bits)), dev(sx), dev(oracle.pack_codes(B, bits)),
                        dev(sw), dev(b) if b is not None else None, bits=bits, K=K,
                        out_dtype=torch.float16 if io == "f16" else torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.epilogue(oracle.gemm_s32(A, B), sx, sw, b, IO_CODE[io])
    got = bits_from_dev(Y)
    ok, maxerr = y_tolerance_ok(got, ref, io)
    assert ok, maxerr
    assert np.array_equal(got, ref)


# Around the launcher's choice between four waves per tile and eight waves per tile (two
# groups splitting the k steps; taken when there are no more tiles than CUs and at least 16
# k steps of 64 bytes): both sides of the tile-count and step-count limits, ragged M and N.
SPLIT_CASES = [(1000, 1040, 1024, 8),    # 36 tiles, 16 steps: split
               (1000, 1040, 896, 8),     # 14 steps: not split
               (770, 2064, 2048, 4),     # 68 tiles, 16 steps of int4: split
               (4096, 2048, 1024, 8),    # exactly 256 tiles: split
               (4096, 2064, 1024, 8)]    # 272 tiles: not split


@pytest.mark.parametrize("M,N,K,bits", SPLIT_CASES)
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_gemm_split_choice_parity(M, N, K, bits, layout):
    need_gpu()
    print("split-choice case M=%d N=%d K=%d bits=%d %s" % (M, N, K, bits, layout), flush=True)
    rng = np.random.default_rng(M + 3 * N + K + bits)
    A = _random_codes(rng, M, K, bits)
    B = _random_codes(rng, N, K, bits)
    packed = oracle.pack_codes(A, bits)
    if layout == "tiled":
        Ad = torch.from_numpy(tile_codes(packed, M, K, bits, pad_fill=0x77)).cuda()
        xl = rq.RQ_X_TILED
    else:
        Ad = torch.from_numpy(packed).cuda()
        xl = rq.RQ_X_ROWS
    Bd = torch.from_numpy(oracle.pack_codes(B, bits)).cuda()
    sx = (rng.random(M) * 0.05).astype(np.float32)
    sw = (rng.random(N) * 2e-4).astype(np.float32)
    b = rng.normal(0, 0.01, N).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).cuda()
    acc = rq.gemm_s32(Ad, Bd, bits=bits, K=K, x_layout=xl, M=M)
    Y = rq.gemm_dequant(Ad, dev(sx), Bd, dev(sw), dev(b), bits=bits, K=K, x_layout=xl)
    torch.cuda.synchronize()
    rows = np.arange(M)
    ref_acc = oracle.gemm_s32(np.ascontiguousarray(A[rows]), B)
    assert np.array_equal(acc.cpu().numpy()[rows], ref_acc)
    assert np.array_equal(bits_from_dev(Y)[rows], oracle.epilogue(ref_acc, sx[rows], sw, b, oracle.F16))


# Around the launcher's choice of eight-wave 256 x 256 tiles (more 256 x 128 tiles than CUs and
# at least 3072 bytes of K): ragged M; N ending on an idle (2176) or a partly filled (2192)
# second half of the last 256-column tile; just below the K limit (2944 bytes: not taken).
N2_CASES = [(4096, 2176, 3072, 8), (4100, 2080, 3072, 8), (4000, 2192, 6144, 4),
            (4096, 2176, 2944, 8)]


@pytest.mark.parametrize("M,N,K,bits", N2_CASES)
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_gemm_n2_choice_parity(M, N, K, bits, layout):
    need_gpu()
    print("n2-choice case M=%d N=%d K=%d bits=%d %s" % (M, N, K, bits, layout), flush=True)
    rng = np.random.default_rng(M + 5 * N + K + bits)
    A = _random_codes(rng, M, K, bits)
    B = _random_codes(rng, N, K, bits)
    packed = oracle.pack_codes(A, bits)
    if layout == "tiled":
        Ad = torch.from_numpy(tile_codes(packed, M, K, bits, pad_fill=0x77)).cuda()
        xl = rq.RQ_X_TILED
    else:
        Ad = torch.from_numpy(packed).cuda()
        xl = rq.RQ_X_ROWS
    Bd = torch.from_numpy(oracle.pack_codes(B, bits)).cuda()
    sx = (rng.random(M) * 0.05).astype(np.float32)
    sw = (rng.random(N) * 2e-4).astype(np.float32)
    b = rng.normal(0, 0.01, N).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).cuda()
    acc = rq.gemm_s32(Ad, Bd, bits=bits, K=K, x_layout=xl, M=M)
    ys = {io: rq.gemm_dequant(Ad, dev(sx), Bd, dev(sw), dev(b), bits=bits, K=K, x_layout=xl,
                              out_dtype=torch.float16 if io == "f16" else torch.bfloat16)
          for io in ("f16", "bf16")}
    torch.cuda.synchronize()
    rows = np.arange(M)
    ref_acc = oracle.gemm_s32(np.ascontiguousarray(A[rows]), B)
    assert np.array_equal(acc.cpu().numpy()[rows], ref_acc)
    for io, Y in ys.items():
        ref = oracle.epilogue(ref_acc, sx[rows], sw, b, IO_CODE[io])
        assert np.array_equal(bits_from_dev(Y)[rows], ref), io


# Shapes with more 256 x 128 tiles than CUs and K of 1024, 1536 or 2048 bytes: with int8 codes
# in the tiled layout and an fp16/bf16 output the launcher loads Xq fragments straight into
# registers (one kernel per K, the k loop unrolled), for the int32 output too; row-major or
# int4 codes take the four-wave LDS kernel. Ragged in M and N; every element compared.
XR_CASES = [(4100, 2064, 1024, 8), (2600, 3088, 1536, 8), (3000, 2960, 2048, 8),
            (4100, 2064, 2048, 4)]


@pytest.mark.parametrize("M,N,K,bits", XR_CASES)
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_gemm_xr_choice_parity(M, N, K, bits, layout):
    need_gpu()
    print("xr-choice case M=%d N=%d K=%d bits=%d %s" % (M, N, K, bits, layout), flush=True)
    rng = np.random.default_rng(M + 3 * N + K + bits)
    A = _random_codes(rng, M, K, bits)
    B = _random_codes(rng, N, K, bits)
    packed = oracle.pack_codes(A, bits)
    if layout == "tiled":
        Ad = torch.from_numpy(tile_codes(packed, M, K, bits, pad_fill=0x77)).cuda()
        xl = rq.RQ_X_TILED
    else:
        Ad = torch.from_numpy(packed).cuda()
        xl = rq.RQ_X_ROWS
    Bd = torch.from_numpy(oracle.pack_codes(B, bits)).cuda()
    sx = (rng.random(M) * 0.05).astype(np.float32)
    sw = (rng.random(N) * 2e-4).astype(np.float32)
    b = rng.normal(0, 0.01, N).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).cuda()
    acc = rq.gemm_s32(Ad, Bd, bits=bits, K=K, x_layout=xl, M=M)
    ys = {io: rq.gemm_dequant(Ad, dev(sx), Bd, dev(sw), dev(b), bits=bits, K=K, x_layout=xl,
                              out_dtype=torch.float16 if io == "f16" else torch.bfloat16)
          for io in ("f16", "bf16")}
    y_nb = rq.gemm_dequant(Ad, dev(sx), Bd, dev(sw), None, bits=bits, K=K, x_layout=xl,
                           out_dtype=torch.float16)
    torch.cuda.synchronize()
    rows = np.arange(M)
    ref_acc = oracle.gemm_s32(np.ascontiguousarray(A[rows]), B)
    assert np.array_equal(acc.cpu().numpy()[rows], ref_acc)
    for io, Y in ys.items():
        ref = oracle.epilogue(ref_acc, sx[rows], sw, b, IO_CODE[io])
        assert np.array_equal(bits_from_dev(Y)[rows], ref), io
    assert np.array_equal(bits_from_dev(y_nb)[rows], oracle.epilogue(ref_acc, sx[rows], sw, None, IO_CODE["f16"]))


# Shapes the launcher sends to the kernel with each CU's weight tile resident in LDS (int8 codes
# in the tiled layout, K = 1024, N = 32 x 96, at least 64 token blocks of 64 per XCD-eighth):
# the smallest such M, ragged M (a partial last block and a partial last 256-row panel), M just
# below the threshold (the next kernel takes it), and several blocks per wave. Every element of
# the int32 accumulators and of both output types is compared.
# Resident-weight kernel (N = 3072 in 96-feature n-tiles; at least 64 token blocks) at ragged M,
# the first M below its threshold, and N = 1024 shapes around the split-K kernel's threshold
# (256 tiles), which the other kernels take.
RW_CASES = [(4096, 3072, 1024), (4100, 3072, 1024), (4033, 3072, 1024), (9999, 3072, 1024),
            (4032, 3072, 1024), (8192, 1024, 1024), (8193, 1024, 1024), (8129, 1024, 1024),
            (12345, 1024, 1024), (8128, 1024, 1024)]


@pytest.mark.parametrize("M,N,K", RW_CASES)
def test_gemm_rw_choice_parity(M, N, K):
    need_gpu()
    print("rw-choice case M=%d N=%d K=%d" % (M, N, K), flush=True)
    rng = np.random.default_rng(M + 7 * N + K)
    A = _random_codes(rng, M, K, 8)
    B = _random_codes(rng, N, K, 8)
    Ad = torch.from_numpy(tile_codes(oracle.pack_codes(A, 8), M, K, 8, pad_fill=0x7F)).cuda()
    Bd = torch.from_numpy(oracle.pack_codes(B, 8)).cuda()
    sx = (rng.random(M) * 0.05).astype(np.float32)
    sw = (rng.random(N) * 2e-4).astype(np.float32)
    b = rng.normal(0, 0.01, N).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).cuda()
    acc = rq.gemm_s32(Ad, Bd, bits=8, K=K, x_layout=rq.RQ_X_TILED, M=M)
    ys = {io: rq.gemm_dequant(Ad, dev(sx), Bd, dev(sw), dev(b), bits=8, K=K, x_layout=rq.RQ_X_TILED,
                              out_dtype=torch.float16 if io == "f16" else torch.bfloat16)
          for io in ("f16", "bf16")}
    y_nb = rq.gemm_dequant(Ad, dev(sx), Bd, dev(sw), None, bits=8, K=K, x_layout=rq.RQ_X_TILED)
    torch.cuda.synchronize()
    ref_acc = oracle.gemm_s32(A, B)
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    for io, Y in ys.items():
        assert np.array_equal(bits_from_dev(Y), oracle.epilogue(ref_acc, sx, sw, b, IO_CODE[io])), io
    assert np.array_equal(bits_from_dev(y_nb), oracle.epilogue(ref_acc, sx, sw, None, IO_CODE["f16"]))


@pytest.mark.parametrize("M,N,K", [(1, 32784, 1024), (300, 16400, 2048), (64, 32784, 1536)])
def test_gemm_xr_few_rows_many_tiles(M, N, K):
    """Xq fragments in registers with one or two token panels spread over more tiles than CUs:
    the panel's pad rows are loaded and multiplied but never stored. Every element compared."""
    need_gpu()
    print("xr-few-rows case M=%d N=%d K=%d" % (M, N, K), flush=True)
    rng = np.random.default_rng(M + N + K)
    A = _random_codes(rng, M, K, 8)
    B = _random_codes(rng, N, K, 8)
    Ad = torch.from_numpy(tile_codes(oracle.pack_codes(A, 8), M, K, 8, pad_fill=0x81)).cuda()
    Bd = torch.from_numpy(oracle.pack_codes(B, 8)).cuda()
    sx = (rng.random(M) * 0.05).astype(np.float32)
    sw = (rng.random(N) * 2e-4).astype(np.float32)
    b = rng.normal(0, 0.01, N).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).cuda()
    Y = rq.gemm_dequant(Ad, dev(sx), Bd, dev(sw), dev(b), bits=8, K=K, x_layout=rq.RQ_X_TILED,
                        out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.epilogue(oracle.gemm_s32(A, B), sx, sw, b, IO_CODE["bf16"])
    assert np.array_equal(bits_from_dev(Y), ref)


# Shapes the launcher sends to its 128-byte-row 256 x 256-tile kernel (row-major codes, K of
# 1536-3071 bytes and at least 192 such tiles), ragged in M and N; every element compared.
WIDE_CASES = [(2048, 6144, 1536, 8), (1900, 6160, 1536, 8), (2000, 6144, 3072, 4)]


@pytest.mark.parametrize("M,N,K,bits", WIDE_CASES)
def test_gemm_wide_tiles_parity(M, N, K, bits):
    need_gpu()
    assert ((M + 255) // 256) * ((N + 255) // 256) >= 192 and 1536 <= K * bits // 8 < 3072
    rng = np.random.default_rng(M + N + K + bits)
    A = _random_codes(rng, M, K, bits)
    B = _random_codes(rng, N, K, bits)
    rows = np.arange(M)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    Ad, Bd = dev(oracle.pack_codes(A, bits)), dev(oracle.pack_codes(B, bits))
    acc = rq.gemm_s32(Ad, Bd, bits=bits, K=K)
    sx = (rng.random(M) * 0.05).astype(np.float32)
    sw = (rng.random(N) * 2e-4).astype(np.float32)
    b = rng.normal(0, 0.01, N).astype(np.float32)
    ys = {io: rq.gemm_dequant(Ad, dev(sx), Bd, dev(sw), dev(b), bits=bits, K=K,
                              out_dtype=torch.float16 if io == "f16" else torch.bfloat16)
          for io in ("f16", "bf16")}
    torch.cuda.synchronize()
    ref_acc = oracle.gemm_s32(A[rows], B)
    assert np.array_equal(acc.cpu().numpy()[rows], ref_acc)
    for io, Y in ys.items():
        ref = oracle.epilogue(ref_acc, sx[rows], sw, b, IO_CODE[io])
        assert np.array_equal(bits_from_dev(Y)[rows], ref), io


def _linear_case(xb, io, W, b, bits):
    Wd = dev_from_bits(W, "f32")
    Wq, ws = rq.quantize_weights(Wd, bits=bits)
    Xd = dev_from_bits(xb, io)
    bd = torch.from_numpy(b).cuda() if b is not None else None
    Y = rq.rotq_linear(Xd, Wq, ws, bd, bits=bits)
    torch.cuda.synchronize()
    wc, _, wsr = oracle.quantize_weights(W, bits)
    ref = oracle.rotq_linear(xb, IO_CODE[io], wc, wsr, b, bits)
    return bits_from_dev(Y), ref["Y"], Wq, ws, wsr


@pytest.mark.parametrize("key", list(synth.CONFIGS))
@pytest.mark.parametrize("M", [1, 77, 333])
def test_rotq_linear_parity_small(key, M):
    need_gpu()
    g = synth.generate(key, M=M)
    cfg = g["cfg"]
    for lin in cfg.linears:
        xb = g["x_bits"] if lin.source == "x" else g["x2_bits"][lin.name]
        got, ref, _, ws, wsr = _linear_case(xb, cfg.io, g["W"][lin.name], g["bias"][lin.name], cfg.bits)
        assert np.array_equal(ws.cpu().numpy(), wsr)
        ok, maxerr = y_tolerance_ok(got, ref, cfg.io)
        assert ok, (lin.name, maxerr)
        assert np.array_equal(got, ref), lin.name


def test_rotq_linear_no_bias_and_zero_rows():
    need_gpu()
    rng = np.random.default_rng(5)
    x = synth.random_rows(rng, 40, 512, "normal", 3, 50.0)
    x[[0, 17, 39]] = 0
    W = rng.normal(0, 0.02, (48, 512)).astype(np.float32)
    W[5] = 0
    b = rng.normal(0, 0.01, 48).astype(np.float32)
    for bias in (b, None):
        got, ref, *_ = _linear_case(synth.to_io_bits(x, "f16"), "f16", W, bias, 8)
        assert np.array_equal(got, ref)
    got, ref, *_ = _linear_case(synth.to_io_bits(x, "f16"), "f16", W, b, 8)
    assert np.array_equal(got[17], b.astype(np.float16).view(np.uint16))   # zero X row -> bias


def test_fp16_overflow_matches_oracle():
    # Round-to-nearest-even with overflow to +-inf on the fp16 store.
    need_gpu()
    rng = np.random.default_rng(6)
    x = synth.random_rows(rng, 8, 256, "normal", 0, 1.0)
    W = rng.normal(0, 0.02, (32, 256)).astype(np.float32)
    b = np.full(32, 65519.0, np.float32)
    b[::2] = -70000.0
    got, ref, *_ = _linear_case(synth.to_io_bits(x, "f16"), "f16", W, b, 8)
    assert np.array_equal(got, ref)
    assert np.isinf(got.view(np.float16)[:, ::2]).all()


def test_deterministic_bits():
    need_gpu()
    g = synth.generate("dit", M=1000, with_second_layer=False)
    W = dev_from_bits(g["W"]["qkv"], "f32")
    Wq, ws = rq.quantize_weights(W)
    X = dev_from_bits(g["x_bits"], "bf16")
    y1 = rq.rotq_linear(X, Wq, ws)
    y2 = rq.rotq_linear(X, Wq, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_runtime_errors_are_raised():
    need_gpu()
    X = torch.zeros(16, 1000, dtype=torch.float16, device="cuda")
    with pytest.raises(rq.ConvRotError) as e:
        rq.rotate_quantize(X)
    assert e.value.status == rq.RQ_EUNSUPPORTED
    Wq = torch.zeros(32, 128, dtype=torch.int8, device="cuda")
    ws = torch.zeros(32, dtype=torch.float32, device="cuda")
    X = torch.zeros(16, 128, dtype=torch.float16, device="cuda")
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):                 # the wrapper checks the size first
        rq.rotq_linear(X, Wq, ws, workspace=small)
    # The C entry point itself returns RQ_EWORKSPACE for the same call.
    Y = torch.empty((16, 32), dtype=torch.float16, device="cuda")
    st = rq.rq_rotq_linear(X.data_ptr(), rq.RQ_F16, 16, 128, Wq.data_ptr(), ws.data_ptr(), 32, None,
                           rq.make_cfg(8), Y.data_ptr(), small.data_ptr(), 64,
                           torch.cuda.current_stream().cuda_stream)
    assert st == rq.RQ_EWORKSPACE


def _edge_rows(K, io, bits):
    """Rows at the reciprocal-overflow edge of the zero-row rule: one-hot rows of magnitude a
    just at and just above the largest a whose fl(q_max / a) is +inf, their negatives, the
    smallest normal, a tiny but quantizable row and an ordinary one. bf16 rows round the edge
    values to bf16 (the first at or below it, the first above)."""
    from tests.test_oracle_quant import _inv_overflow_edge
    qmax = 127 if bits == 8 else 7
    a_lo, a_hi = _inv_overflow_edge(qmax)
    if io == "bf16":
        lo_b = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(np.array([a_lo], np.float32)))[0]
        while lo_b > a_lo:
            lo_b = np.float32(np.uint32(lo_b.view(np.uint32) - (1 << 16)).view(np.float32))
        a_lo, a_hi = lo_b, np.float32(np.uint32(lo_b.view(np.uint32) + (1 << 16)).view(np.float32))
    rng = np.random.default_rng(K + bits)
    x = np.zeros((8, K), np.float32)
    x[0, 0], x[1, 5], x[2, 0], x[3, K - 1] = a_lo, -a_lo, a_hi, -a_hi
    x[4, 7] = np.float32(2.0 ** -126)
    x[5] = rng.normal(0, 1, K).astype(np.float32) * np.float32(1e-30)
    x[6] = rng.normal(0, 1, K).astype(np.float32)
    x[7, :130] = a_lo                      # rotates to a block absmax above the edge
    return x if io == "f32" else synth.to_io_bits(x, io)


@pytest.mark.parametrize("K", [256, 1024, 2176])
@pytest.mark.parametrize("io,bits", [("f32", 8), ("f32", 4), ("bf16", 8), ("bf16", 4)])
def test_reciprocal_overflow_rows(K, io, bits):
    """The zero-row rule (a row whose fl(q_max / a) is +inf gets scale 0 and codes 0) on the
    activation quantizer, fast and generic kernels, and on the weight quantizer's three rules."""
    need_gpu()
    xb = _edge_rows(K, io, bits)
    Xd = dev_from_bits(xb, io)
    ref_c, ref_s, ref_p = oracle.quantize_rows(xb, IO_CODE[io], bits, want_pre=True)
    assert ref_s[0] == 0 and ref_s[2] > 0
    Xq, xs = rq.rotate_quantize(Xd, bits=bits)
    torch.cuda.synchronize()
    assert compare_codes(codes_np(Xq), ref_c, ref_p, bits, K) == 0
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    for mode in (rq.RQ_W_ABSMAX, rq.RQ_W_MSE):
        Wq, ws = rq.quantize_weights(Xd, bits=bits, w_scale_mode=mode)
        torch.cuda.synchronize()
        if mode == rq.RQ_W_MSE:
            c, s, _, _ = oracle.quantize_rows_mse(xb, IO_CODE[io], bits)
        else:
            c, s = ref_c, ref_s
        assert np.array_equal(codes_np(Wq).view(np.uint8), oracle.pack_codes(c, bits).view(np.uint8)), mode
        assert np.array_equal(ws.cpu().numpy().view(np.uint32), s.view(np.uint32)), mode
    # Tensor-wise: a tensor of edge rows only (its absmax below, then above, the edge).
    for rows in ([0, 1], [0, 1, 2]):
        sub = np.ascontiguousarray(xb[rows])
        Wq, ws = rq.quantize_weights(dev_from_bits(sub, io), bits=bits, w_scale_mode=rq.RQ_W_TENSOR)
        torch.cuda.synchronize()
        c, s, _ = oracle.quantize_tensorwise(sub, IO_CODE[io], bits)
        assert np.array_equal(codes_np(Wq).view(np.uint8), oracle.pack_codes(c, bits).view(np.uint8)), rows
        assert np.array_equal(ws.cpu().numpy().view(np.uint32), s.view(np.uint32)), rows
