"""MI355X-native ConvRot quantized linear (W8A8 / W4A4).

The compute lives in ``libconvrot.so`` -- hand-written HIP for gfx950 behind the C ABI
declared in ``include/convrot.h``; ``binding`` marshals tensors into it. Importing the package
does not load the library; the first call does, and raises if it has not been built.
"""
from .binding import (  # noqa: F401
    ConvRotError, RQ_ACT_GELU_ERF, RQ_ACT_GELU_TANH, RQ_ACT_NONE, RQ_BF16, RQ_EHIP, RQ_EINVAL,
    RQ_EUNSUPPORTED, RQ_EWORKSPACE, RQ_F16, RQ_F32, RQ_NOALLOC_SCRATCH_BYTES,
    RQ_OK, RQ_ROT_WHT, RQ_W_ABSMAX, RQ_W_FP6, RQ_W_MSE, RQ_W_ROWS, RQ_W_TENSOR, RQ_X_FP6, RQ_X_ROWS,
    RQ_X_TILED, code_shape, gemm_dequant, gemm_s32, lib_path, load,
    make_cfg, rq_codes_bytes, rq_weight_bytes,
    quantize_weights, rotate_quantize, rotq_linear, rq_check_rotq_linear_args, rq_gemm_dequant,
    rq_gemm_s32, rq_qconfig, rq_quantize_weights, rq_rotate_quantize, rq_rotq_linear,
    rq_rotq_linear_noalloc,
    rq_rotq_linear_workspace_size, rq_status_string, workspace_size,
)
