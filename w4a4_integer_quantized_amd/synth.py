"""Seeded synthetic workloads for the ConvRot quantized linear (inputs only).

This module draws inputs and nothing else: it holds none of the method's arithmetic (no
rotation, quantization, integer GEMM or dequantization). The tests, the smoke check and the
benchmark take their inputs from here, and both the HIP path and the CPU oracle consume the
same arrays.

The pages measure on SAM 3.1 (a ViT image encoder at 1008-pixel input) and TRELLIS.2 (a
diffusion transformer); no checkpoint, image or dataset is used. These shapes and value
distributions stand in for those workloads' eligible block linears:

  single      single linear          X f16 [256, 1024], N(0,1), 8 outlier channels x50, W [1024, 1024]
  vit_mlp     ViT-L MLP pair, b=1    X f16 [5184, 1024], N(0,1), 1% outlier channels x30;
                             fc1 W [4096, 1024], fc2 W [1024, 4096] (input: erf-GELU of an
                             fc1-shaped activation)
  vit_attn    ViT-L attention, b=8   X f16 [41472, 1024], N(0,1), 8 outlier channels x50;
                             qkv W [3072, 1024] and out-proj W [1024, 1024], both on X
  w4a4        W4A4 linear            X f16 [5184, 4096], Laplace(0,1), 1% outlier channels x30,
                             W [1024, 4096], int4 weights and activations
  dit         DiT block, bf16 I/O    X bf16 [8192, 1536], N(0,1), 16 outlier channels x50;
                             qkv W [4608, 1536], W1 [6144, 1536], W2 [1536, 6144] (input:
                             tanh-GELU of a W1-shaped activation)

Every weight is N(0, 0.02) fp32 and every bias N(0, 0.01) fp32. Draw order from
numpy.random.default_rng(seed) (PCG64): outlier channel indices, X body, each W in listed
order, each bias, then the second-layer activation body of an MLP pair. Outlier channels are
the same columns for every token. X is rounded to f16 (IEEE round-to-nearest-even) or bf16
(round-to-nearest-even of the upper 16 bits).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Linear:
    name: str
    N: int                 # output features (rows of W)
    K: int                 # input features
    source: str            # "x" (the config's X) or "gelu_erf" / "gelu_tanh" (second layer)
    producer: str = ""     # second layer: the linear whose output (through GELU) feeds this one


@dataclasses.dataclass(frozen=True)
class Config:
    key: str
    workload: str
    seed: int
    M: int
    K: int
    x_dist: str            # "normal" | "laplace"
    n_outliers: int
    outlier_scale: float
    io: str                # "f16" | "bf16"
    bits: int              # 8 (W8A8) or 4 (W4A4)
    linears: tuple


CONFIGS: Dict[str, Config] = {
    "single": Config("single", "w8a8_single_linear_256x1024x1024", 0, 256, 1024, "normal", 8, 50.0,
                 "f16", 8, (Linear("linear", 1024, 1024, "x"),)),
    "vit_mlp": Config("vit_mlp", "vitl_mlp_pair_b1_5184x1024x4096", 1, 5184, 1024, "normal", 10, 30.0,
                 "f16", 8, (Linear("fc1", 4096, 1024, "x"), Linear("fc2", 1024, 4096, "gelu_erf", "fc1"))),
    "vit_attn": Config("vit_attn", "vitl_attn_proj_b8_41472x1024_qkv3072_oproj1024", 2, 41472, 1024,
                 "normal", 8, 50.0, "f16", 8,
                 (Linear("qkv", 3072, 1024, "x"), Linear("oproj", 1024, 1024, "x"))),
    "w4a4": Config("w4a4", "w4a4_linear_5184x4096x1024", 3, 5184, 4096, "laplace", 41, 30.0,
                 "f16", 4, (Linear("linear", 1024, 4096, "x"),)),
    "dit": Config("dit", "dit_block_bf16_8192x1536", 4, 8192, 1536, "normal", 16, 50.0, "bf16", 8,
                 (Linear("qkv", 4608, 1536, "x"), Linear("w1", 6144, 1536, "x"),
                  Linear("w2", 1536, 6144, "gelu_tanh", "w1"))),
}


def _check_configs():
    for cfg in CONFIGS.values():
        names = {lin.name: lin for lin in cfg.linears}
        for lin in cfg.linears:
            if lin.source == "x":
                assert lin.K == cfg.K and not lin.producer, (cfg.key, lin.name)
            else:
                prod = names[lin.producer]
                assert prod.source == "x" and prod.N == lin.K, (cfg.key, lin.name)


_check_configs()


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Input preparation: round float32 to bfloat16 (nearest, ties to even) as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def to_io_bits(x: np.ndarray, io: str) -> np.ndarray:
    """float32 -> raw uint16 bits of the config's I/O dtype."""
    if io == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    if io == "bf16":
        return f32_to_bf16_bits_rne(x)
    raise ValueError(io)


def gelu(z: np.ndarray, kind: str) -> np.ndarray:
    """GELU in float64 (erf or tanh form), for making second-layer inputs and error context."""
    return _gelu(z, kind)


def _gelu(z: np.ndarray, kind: str) -> np.ndarray:
    z = z.astype(np.float64)
    if kind == "gelu_erf":
        from scipy.special import erf
        return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def make_x(rng: np.random.Generator, M: int, K: int, dist: str, n_out: int, scale: float):
    idx = rng.choice(K, n_out, replace=False) if n_out > 0 else np.zeros(0, np.int64)
    if dist == "normal":
        x = rng.standard_normal((M, K), dtype=np.float32)
    elif dist == "laplace":
        x = rng.laplace(0.0, 1.0, (M, K)).astype(np.float32)
    else:
        raise ValueError(dist)
    if n_out:
        x[:, idx] *= np.float32(scale)
    return x, np.sort(idx)


def generate(key: str, M: Optional[int] = None, with_second_layer: bool = True) -> dict:
    """All inputs of one configuration.

    M overrides the token count (same draw recipe, fewer rows) for small parity cases.
    Returns {"cfg", "x_bits" uint16 [M, K] (raw f16/bf16 bits), "outliers",
             "W": {name: f32 [N, K]}, "bias": {name: f32 [N]},
             "x2_bits": {name: uint16 [M, K2]} for second-layer linears}.
    """
    cfg = CONFIGS[key]
    M = cfg.M if M is None else M
    rng = np.random.default_rng(cfg.seed)
    x, idx = make_x(rng, M, cfg.K, cfg.x_dist, cfg.n_outliers, cfg.outlier_scale)
    W, bias = {}, {}
    for lin in cfg.linears:
        W[lin.name] = rng.normal(0.0, 0.02, (lin.N, lin.K)).astype(np.float32)
    for lin in cfg.linears:
        bias[lin.name] = rng.normal(0.0, 0.01, (lin.N,)).astype(np.float32)
    x_bits = to_io_bits(x, cfg.io)
    out = {"cfg": cfg, "x_bits": x_bits, "outliers": idx, "W": W, "bias": bias, "x2_bits": {}}
    if with_second_layer:
        # Activation of the first MLP layer: its pre-GELU values have variance
        # 0.02^2 * sum_k E[x_k^2] (N(0, 0.02) weights against the outlier-scaled X).
        ex2 = 2.0 if cfg.x_dist == "laplace" else 1.0
        var = 0.02 ** 2 * ex2 * ((cfg.K - cfg.n_outliers) + cfg.n_outliers * cfg.outlier_scale ** 2)
        for lin in cfg.linears:
            if lin.source != "x":
                z = rng.normal(0.0, math.sqrt(var), (M, lin.K))
                out["x2_bits"][lin.name] = to_io_bits(_gelu(z, lin.source).astype(np.float32), cfg.io)
    return out


def random_rows(rng: np.random.Generator, rows: int, K: int, dist: str = "normal",
                n_out: int = 0, scale: float = 1.0) -> np.ndarray:
    """A small float32 [rows, K] block for edge-case tests."""
    x, _ = make_x(rng, rows, K, dist, n_out, scale)
    return x


def linears(key: str) -> List[Linear]:
    return list(CONFIGS[key].linears)
