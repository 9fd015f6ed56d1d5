"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and
validates arguments on the host before any launch (no GPU needed for any of these)."""
import ctypes
import os
import re

import numpy as np
import pytest

import w4a4_integer_quantized_amd as rq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")

A = 0x10000          # fake, 16-byte aligned "device addresses": only compared, never touched
GB = 1 << 30


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = rq.load()
    names = declared_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert lib.rq_version().decode().count(".") == 2


def test_status_strings():
    for s in range(5):
        assert rq.rq_status_string(s).startswith("RQ_")


def _args(**kw):
    cfg = rq.make_cfg(kw.pop("bits", 8), kw.pop("rot", 128), kw.pop("kind", rq.RQ_ROT_WHT),
                      kw.pop("x_layout", rq.RQ_X_ROWS))
    M, K, N = kw.pop("M", 256), kw.pop("K", 1024), kw.pop("N", 1024)
    base = dict(X=A, x_dtype=rq.RQ_F16, M=M, K=K, Wq=A + 4 * GB, w_scale=A + 8 * GB, N=N,
                bias=A + 9 * GB, cfg=cfg, Y=A + 12 * GB, ws=A + 20 * GB,
                ws_bytes=rq.rq_rotq_linear_workspace_size(M, K, cfg))
    base.update(kw)
    return base


def check(**kw):
    a = _args(**kw)
    return rq.rq_check_rotq_linear_args(a["X"], a["x_dtype"], a["M"], a["K"], a["Wq"], a["w_scale"],
                                        a["N"], a["bias"], a["cfg"], a["Y"], a["ws"], a["ws_bytes"])


def test_valid_arguments_pass():
    assert check() == rq.RQ_OK
    assert check(bias=None) == rq.RQ_OK
    assert check(M=0) == rq.RQ_OK
    assert check(bits=4, K=4096) == rq.RQ_OK
    assert check(bits=4, K=384) == rq.RQ_OK
    assert check(K=131072, N=16) == rq.RQ_OK
    assert check(x_dtype=rq.RQ_BF16, K=1536, N=4608) == rq.RQ_OK
    assert check(M=41472, K=1024, N=3072) == rq.RQ_OK


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), rq.RQ_EINVAL),
    (dict(Y=None), rq.RQ_EINVAL),
    (dict(Wq=A + 4 * GB + 8), rq.RQ_EINVAL),                 # misaligned
    (dict(w_scale=None), rq.RQ_EINVAL),
    (dict(M=-1), rq.RQ_EINVAL),
    (dict(x_dtype=7), rq.RQ_EINVAL),
    (dict(x_dtype=rq.RQ_F32), rq.RQ_EUNSUPPORTED),
    (dict(K=1000), rq.RQ_EUNSUPPORTED),
    (dict(K=64), rq.RQ_EUNSUPPORTED),
    (dict(K=131072 + 128), rq.RQ_EUNSUPPORTED),
    (dict(N=1000), rq.RQ_EUNSUPPORTED),
    (dict(N=0), rq.RQ_EUNSUPPORTED),
    (dict(bits=6), rq.RQ_EUNSUPPORTED),
    (dict(rot=64), rq.RQ_EUNSUPPORTED),
    (dict(x_layout=3), rq.RQ_EINVAL),
    (dict(x_layout=rq.RQ_X_FP6), rq.RQ_EUNSUPPORTED),           # FP6 codes are 4-bit only
    (dict(kind=0), rq.RQ_EUNSUPPORTED),
    (dict(ws_bytes=100), rq.RQ_EWORKSPACE),
    (dict(Y=A + 100 * 2), rq.RQ_EINVAL),                      # Y overlaps X
    (dict(ws=A + 12 * GB + 4096), rq.RQ_EINVAL),              # workspace overlaps Y
    (dict(ws=A + 64), rq.RQ_EINVAL),                          # workspace overlaps X
])
def test_invalid_arguments_rejected(kw, status):
    assert check(**kw) == status
    assert rq.load().rq_last_error_detail().decode()


def test_workspace_size():
    # Tiled codes: rows padded to whole 256-row panels, then x_scale; each part 256-byte aligned.
    cfg8, cfg4 = rq.make_cfg(8), rq.make_cfg(4)
    assert rq.rq_rotq_linear_workspace_size(256, 1024, cfg8) == 256 * 1024 + 1024
    assert rq.rq_rotq_linear_workspace_size(5184, 4096, cfg4) == 5376 * 2048 + 5184 * 4
    assert rq.rq_rotq_linear_workspace_size(5, 256, cfg4) == 256 * 128 + 256
    assert rq.rq_rotq_linear_workspace_size(3, 128, cfg8) == 256 * 128 + 256
    assert rq.rq_rotq_linear_workspace_size(0, 1024, cfg8) == 0
    assert rq.rq_rotq_linear_workspace_size(3, 128, rq.make_cfg(5)) == 0
    # The layout field of cfg does not change the fused call's workspace.
    assert rq.rq_rotq_linear_workspace_size(300, 1024, rq.make_cfg(8, x_layout=rq.RQ_X_TILED)) == \
        rq.rq_rotq_linear_workspace_size(300, 1024, cfg8)


def test_codes_bytes():
    rows, tiled = rq.make_cfg(8), rq.make_cfg(8, x_layout=rq.RQ_X_TILED)
    assert rq.rq_codes_bytes(300, 1024, rows) == 300 * 1024
    assert rq.rq_codes_bytes(300, 1024, tiled) == 512 * 1024
    assert rq.rq_codes_bytes(256, 1024, tiled) == 256 * 1024
    assert rq.rq_codes_bytes(1, 4096, rq.make_cfg(4, x_layout=rq.RQ_X_TILED)) == 256 * 2048
    assert rq.rq_codes_bytes(7, 4096, rq.make_cfg(4)) == 7 * 2048
    assert rq.rq_codes_bytes(0, 1024, tiled) == 0
    assert rq.rq_codes_bytes(5, 1000, rows) == 0                       # K % 128 != 0
    assert rq.rq_codes_bytes(5, 1024, rq.make_cfg(8, x_layout=3)) == 0  # bad layout
    # FP6 tiles: 48 bytes per 64 codes, rows padded to 256 (activations) or 128 (weights).
    fp6x = rq.make_cfg(4, x_layout=rq.RQ_X_FP6)
    assert rq.rq_codes_bytes(300, 1024, fp6x) == 512 * 16 * 48
    assert rq.rq_codes_bytes(5, 1024, rq.make_cfg(8, x_layout=rq.RQ_X_FP6)) == 0   # 8-bit codes
    fp6w = rq.make_cfg(4, w_layout=rq.RQ_W_FP6)
    assert rq.rq_weight_bytes(100, 256, fp6w) == 128 * 4 * 48
    assert rq.rq_weight_bytes(100, 256, rq.make_cfg(4)) == 100 * 128
    assert rq.rq_weight_bytes(100, 256, rq.make_cfg(8)) == 100 * 256
    assert rq.rq_weight_bytes(100, 256, rq.make_cfg(8, w_layout=rq.RQ_W_FP6)) == 0
    # The fused call's workspace follows the weight layout.
    assert rq.rq_rotq_linear_workspace_size(300, 1024, fp6w) == 512 * 16 * 48 + 1280


def test_entry_points_reject_before_launch():
    # Invalid calls must return a status without touching the (absent) GPU.
    cfg = rq.make_cfg(8)
    assert rq.rq_quantize_weights(A, rq.RQ_F32, 16, 100, cfg, A + GB, A + 2 * GB, None) == rq.RQ_EUNSUPPORTED
    assert rq.rq_rotate_quantize(A, 9, 16, 128, cfg, A + GB, A + 2 * GB, None) == rq.RQ_EINVAL
    assert rq.rq_rotate_quantize(A, rq.RQ_F16, 16, 128, cfg, A + 8, A + 2 * GB, None) == rq.RQ_EINVAL  # overlap
    assert rq.rq_gemm_dequant(A, A + GB, A + 2 * GB, A + 3 * GB, None, 16, 24, 128, cfg, A + 4 * GB,
                              rq.RQ_F16, None) == rq.RQ_EUNSUPPORTED   # N % 16
    assert rq.rq_gemm_dequant(A, A + GB, A + 2 * GB, A + 3 * GB, None, 16, 32, 128, cfg, A + 4 * GB,
                              rq.RQ_F32, None) == rq.RQ_EUNSUPPORTED   # f32 output
    assert rq.rq_gemm_s32(A, A + GB, 16, 32, 128, rq.make_cfg(3), A + 2 * GB, None) == rq.RQ_EUNSUPPORTED
    assert rq.rq_gemm_s32(A, A + GB, 16, 32, 128, cfg, A + 8, None) == rq.RQ_EINVAL     # misaligned/overlap
    # M == 0 is a no-op that succeeds without launching anything
    assert rq.rq_gemm_s32(A, A + GB, 0, 32, 128, cfg, A + 2 * GB, None) == rq.RQ_OK
    assert rq.rq_rotate_quantize(A, rq.RQ_F16, 0, 128, cfg, A + GB, A + 2 * GB, None) == rq.RQ_OK
    # The weight-scale rule is validated for every entry point; N == 0 is a no-op in each rule.
    bad = rq.make_cfg(8, w_scale_mode=3)
    assert rq.rq_quantize_weights(A, rq.RQ_F32, 16, 128, bad, A + GB, A + 2 * GB, None) == rq.RQ_EINVAL
    assert rq.rq_gemm_s32(A, A + GB, 16, 32, 128, bad, A + 2 * GB, None) == rq.RQ_EINVAL
    # FP6 activation codes need FP6 weight codes in the GEMM entry points, and vice versa.
    fx = rq.make_cfg(4, x_layout=rq.RQ_X_FP6)
    fw = rq.make_cfg(4, w_layout=rq.RQ_W_FP6)
    assert rq.rq_gemm_s32(A, A + GB, 16, 32, 128, fx, A + 2 * GB, None) == rq.RQ_EINVAL
    assert rq.rq_gemm_s32(A, A + GB, 16, 32, 128, fw, A + 2 * GB, None) == rq.RQ_EINVAL
    assert rq.rq_quantize_weights(A, rq.RQ_F32, 16, 128, rq.make_cfg(8, w_layout=rq.RQ_W_FP6), A + GB,
                                  A + 2 * GB, None) == rq.RQ_EUNSUPPORTED
    assert rq.rq_quantize_weights(A, rq.RQ_F32, 16, 128, rq.make_cfg(4, w_layout=2), A + GB,
                                  A + 2 * GB, None) == rq.RQ_EINVAL
    # The epilogue activation is validated for every entry point (M == 0 launches nothing).
    for act in (rq.RQ_ACT_NONE, rq.RQ_ACT_GELU_ERF, rq.RQ_ACT_GELU_TANH):
        c = rq.make_cfg(8, act=act)
        assert rq.rq_gemm_dequant(A, A + GB, A + 2 * GB, A + 3 * GB, None, 0, 32, 128, c, A + 4 * GB,
                                  rq.RQ_F16, None) == rq.RQ_OK
        assert rq.rq_check_rotq_linear_args(A, rq.RQ_F16, 16, 128, A + GB, A + 2 * GB, 32, None, c,
                                            A + 3 * GB, A + 4 * GB, 1 << 20) == rq.RQ_OK
    for act in (-1, 3):
        c = rq.make_cfg(8, act=act)
        assert rq.rq_gemm_dequant(A, A + GB, A + 2 * GB, A + 3 * GB, None, 16, 32, 128, c, A + 4 * GB,
                                  rq.RQ_F16, None) == rq.RQ_EINVAL
        assert rq.rq_check_rotq_linear_args(A, rq.RQ_F16, 16, 128, A + GB, A + 2 * GB, 32, None, c,
                                            A + 3 * GB, A + 4 * GB, 1 << 20) == rq.RQ_EINVAL
    for mode in (rq.RQ_W_ABSMAX, rq.RQ_W_MSE, rq.RQ_W_TENSOR):
        c = rq.make_cfg(4, w_scale_mode=mode)
        assert rq.rq_quantize_weights(A, rq.RQ_F32, 0, 256, c, A + GB, A + 2 * GB, None) == rq.RQ_OK
        assert rq.rq_quantize_weights(A, rq.RQ_F32, 16, 200, c, A + GB, A + 2 * GB, None) == rq.RQ_EUNSUPPORTED


def test_tensor_wrappers_refuse_host_tensors():
    import torch
    with pytest.raises(ValueError):
        rq.rotate_quantize(torch.zeros(4, 128, dtype=torch.float16))


def test_qconfig_struct_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} rq_qconfig;", text, re.S).group(1)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert [f for f, _ in rq.rq_qconfig._fields_] == fields
    assert ctypes.sizeof(rq.rq_qconfig) == 4 * len(fields)


def test_fp6_test_helpers_follow_e2m3():
    """The tests' FP6 encoder/decoder against the E2M3 definition: every code in [-7, 7] maps to
    the pattern whose value (sign, 2-bit exponent with bias 1, 3-bit mantissa) is the code."""
    from tests.gpu_util import _FP6_MAG, _FP6_VALUE, fp6_tile, fp6_untile
    for q in range(8):
        p = int(_FP6_MAG[q])
        e, m = (p >> 3) & 3, p & 7
        assert (m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1 + m / 8.0)) == q
        assert _FP6_VALUE[p] == q and _FP6_VALUE[p | 32] == -q
    rng = np.random.default_rng(0)
    c = rng.integers(-7, 8, (300, 384)).astype(np.int8)
    for P in (128, 256):
        t = fp6_tile(c, P)
        assert t.size == (300 + P - 1) // P * P * 6 * 48
        assert np.array_equal(fp6_untile(t, 300, 384, P), c)


# ---- the tensor wrappers' own checks (the C ABI sees only pointers, so shapes, dtypes and
# buffer sizes are checked in Python before any device access; CPU tensors suffice here) ----
def _torch_cpu_args(M=64, K=256, N=32, bits=8):
    import torch
    X = torch.zeros((M, K), dtype=torch.float16)
    Wq = torch.zeros((N, K if bits == 8 else K // 2), dtype=torch.int8 if bits == 8 else torch.uint8)
    return X, Wq, torch.zeros(N), torch.zeros(N)


@pytest.mark.parametrize("bad", ["w_scale_f16", "w_scale_len", "bias_f16", "bias_len", "wq_other_k",
                                 "wq_other_bits", "out_shape", "out_dtype", "x_f32", "x_3d", "ws_small"])
def test_rotq_linear_wrapper_rejects_bad_buffers(bad):
    import torch
    X, Wq, ws, b = _torch_cpu_args()
    kw = {}
    if bad == "w_scale_f16":
        ws = ws.half()
    elif bad == "w_scale_len":
        ws = torch.zeros(48)
    elif bad == "bias_f16":
        b = b.half()
    elif bad == "bias_len":
        b = torch.zeros(16)
    elif bad == "wq_other_k":
        Wq = torch.zeros((32, 512), dtype=torch.int8)
    elif bad == "wq_other_bits":
        kw["bits"] = 4                         # int8 [N, K] is twice the bytes of 4-bit codes
    elif bad == "out_shape":
        kw["out"] = torch.empty((64, 16), dtype=torch.float16)
    elif bad == "out_dtype":
        kw["out"] = torch.empty((64, 32), dtype=torch.bfloat16)
    elif bad == "x_f32":
        X = X.float()
    elif bad == "x_3d":
        X = X.view(4, 16, 256)
    elif bad == "ws_small":
        kw["workspace"] = torch.empty((100,), dtype=torch.uint8)
    with pytest.raises(ValueError):
        rq.rotq_linear(X, Wq, ws, b, **kw)


def test_gemm_wrappers_reject_bad_buffers():
    import torch
    Wq = torch.zeros((32, 256), dtype=torch.int8)
    Xq = torch.zeros((64, 256), dtype=torch.int8)
    xs, ws = torch.zeros(64), torch.zeros(32)
    with pytest.raises(ValueError):            # Xq shorter than M rows of codes
        rq.gemm_dequant(Xq[:10], xs, Wq, ws)
    with pytest.raises(ValueError):            # x_scale of the wrong dtype
        rq.gemm_dequant(Xq, xs.double(), Wq, ws)
    with pytest.raises(ValueError):            # w_scale shorter than Wq's rows
        rq.gemm_dequant(Xq, xs, Wq, ws[:16])
    with pytest.raises(ValueError):            # 4-bit codes need half the bytes
        rq.gemm_s32(Xq, Wq, bits=4)
    with pytest.raises(ValueError):            # tiled codes of M rows need the padded size
        rq.gemm_s32(torch.zeros(64 * 256, dtype=torch.uint8), Wq, x_layout=rq.RQ_X_TILED, M=64)
    with pytest.raises(ValueError):            # tiled layout without M
        rq.gemm_s32(Xq, Wq, x_layout=rq.RQ_X_TILED)


def test_wrappers_accept_valid_cpu_buffers_up_to_the_device_check():
    """Valid shapes pass every size check and stop only at the device check."""
    import torch
    X, Wq, ws, b = _torch_cpu_args()
    with pytest.raises(ValueError, match="device tensor"):
        rq.rotq_linear(X, Wq, ws, b, workspace=torch.empty(rq.workspace_size(64, 256), dtype=torch.uint8))
    Xt = torch.zeros(256 * 256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="device tensor"):
        rq.gemm_s32(Xt, Wq, x_layout=rq.RQ_X_TILED, M=64)


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define RQ_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == rq.RQ_NOALLOC_SCRATCH_BYTES
    # every workload's workspace fits it
    from w4a4_integer_quantized_amd import synth
    for cfg in synth.CONFIGS.values():
        for lin in cfg.linears:
            assert rq.workspace_size(cfg.M, lin.K, cfg.bits) <= rq.RQ_NOALLOC_SCRATCH_BYTES, (cfg.key, lin.name)


def test_ceiling_probe_library_loads_and_rejects_bad_arguments():
    """The bench's memory-ceiling probe (libconvrot_ceiling.so): exported, and invalid arguments
    are refused before anything touches a device."""
    import ctypes
    from w4a4_integer_quantized_amd import build as B
    if not os.path.exists(B.CEILING_LIB):
        pytest.skip("libconvrot_ceiling.so not built")
    fn = ctypes.CDLL(B.CEILING_LIB).rqc_hbm_pattern
    fn.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                   ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    p = ctypes.c_void_p(16)
    assert fn(3, p, p, 8, 1024, 1, None) == 1           # unknown mode
    assert fn(0, None, p, 8, 1024, 1, None) == 1        # null input
    assert fn(0, p, p, 0, 1024, 1, None) == 1           # empty
    assert fn(0, p, p, 8, 1000, 1, None) == 1           # K not a multiple of 128
    assert fn(0, p, p, 8, 17 * 128, 1, None) == 1       # 17 blocks: not G * NI
