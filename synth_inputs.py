"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no NVFP4 arithmetic: it only draws random numbers and rounds
them to the input dtypes.  Every tensor comes from
``numpy.random.default_rng([seed, config_id, tensor_id])`` (PCG64): fp32
normals (optionally with a Bernoulli outlier mask scaled in fp32), then
round-to-nearest-even to bf16/fp16 by torch's CPU cast.

Tensor ids: 0 activations, 1 weights / fc1, 2 fc2, 3 router logits,
4 router correction bias, 5 outlier mask.

Workloads (sizes from the pages' use cases, see the design notes):
  C1  quantize + GEMM        B=16,  K=256,  N=256
  C2  decode GEMM            B in {1,4,8}, K=4096, N=8192
  C3  prefill GEMM           B=4096, K=8192, N=8192
  C4  SwiGLU + quantize      [8192, 2*14336] bf16, 1% entries x50
  C5  W4A16 MoE              T=256, E=64, top-8, nGroup=8, topkGroup=4,
                             hidden 2048, inter 1024
"""
from __future__ import annotations

import numpy as np
import torch

SEED = 0

CONFIGS = {
    "C1": dict(B=16, K=256, N=256, a_std=1.0, w_std=0.02),
    "C2": dict(B=(1, 4, 8), K=4096, N=8192, a_std=1.0, w_std=0.02),
    "C3": dict(B=4096, K=8192, N=8192, a_std=1.0, w_std=0.02),
    "C4": dict(rows=8192, H=14336, std=1.0, outlier_frac=0.01, outlier_scale=50.0),
    "C5": dict(T=256, E=64, top_k=8, n_group=8, topk_group=4, hidden=2048, inter=1024,
               logit_std=1.0, bias_std=0.1, x_std=1.0, w_std=0.02, norm_topk_prob=True,
               routed_scaling=1.0),
}
CONFIG_ID = {"C1": 0, "C2": 1, "C3": 2, "C4": 3, "C5": 4}


def rng(config: str | int, tensor_id: int, seed: int = SEED) -> np.random.Generator:
    cid = CONFIG_ID[config] if isinstance(config, str) else int(config)
    return np.random.default_rng([seed, cid, tensor_id])


def normal_f32(shape, std: float, config, tensor_id: int, seed: int = SEED,
               outlier_frac: float = 0.0, outlier_scale: float = 1.0) -> np.ndarray:
    g = rng(config, tensor_id, seed)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if outlier_frac > 0.0:
        m = rng(config, 5, seed).random(size=shape, dtype=np.float32) < outlier_frac
        x[m] *= np.float32(outlier_scale)
    return x


def to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def to_fp16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float16)


def bf16_normal(shape, std, config, tensor_id, seed=SEED, **kw) -> torch.Tensor:
    return to_bf16(normal_f32(shape, std, config, tensor_id, seed, **kw))


def fp16_normal(shape, std, config, tensor_id, seed=SEED, **kw) -> torch.Tensor:
    return to_fp16(normal_f32(shape, std, config, tensor_id, seed, **kw))


def gemm_inputs(config: str, B: int | None = None, seed: int = SEED, K=None, N=None):
    """bf16 activations [B,K] ~ N(0, a_std) and weights [N,K] ~ N(0, w_std)."""
    c = CONFIGS[config]
    B = c["B"] if B is None else B
    K = c["K"] if K is None else K
    N = c["N"] if N is None else N
    a = bf16_normal((B, K), c["a_std"], config, 0, seed)
    w = bf16_normal((N, K), c["w_std"], config, 1, seed)
    return a, w


def swiglu_input(rows=None, H=None, seed: int = SEED, config="C4") -> torch.Tensor:
    c = CONFIGS["C4"]
    rows = c["rows"] if rows is None else rows
    H = c["H"] if H is None else H
    return bf16_normal((rows, 2 * H), c["std"], config, 0, seed,
                       outlier_frac=c["outlier_frac"], outlier_scale=c["outlier_scale"])


def moe_inputs(seed: int = SEED, T=None, E=None, hidden=None, inter=None, weights: bool = True):
    """Router logits/bias (fp32), hidden states (fp16), fc1/fc2 weights (bf16)."""
    c = CONFIGS["C5"]
    T = c["T"] if T is None else T
    E = c["E"] if E is None else E
    hidden = c["hidden"] if hidden is None else hidden
    inter = c["inter"] if inter is None else inter
    logits = normal_f32((T, E), c["logit_std"], "C5", 3, seed)
    bias = normal_f32((E,), c["bias_std"], "C5", 4, seed)
    x = fp16_normal((T, hidden), c["x_std"], "C5", 0, seed)
    w1 = bf16_normal((E * inter, hidden), c["w_std"], "C5", 1, seed) if weights else None
    w2 = bf16_normal((E * hidden, inter), c["w_std"], "C5", 2, seed) if weights else None
    return dict(logits=logits, bias=bias, x=x, w1=w1, w2=w2, T=T, E=E, hidden=hidden, inter=inter)


def random_nvfp4_operands(B: int, N: int, K: int, seed: int = SEED, config: int = 60) -> dict:
    """Arbitrary valid GEMM operands drawn directly in the stored formats (no
    quantization involved): uniform code bytes, positive finite combined
    activation scales with a uniform exponent in [-10, 2] and uniform
    mantissa bits, E4M3 weight scale bytes 0x00..0x7E (positive, finite) and
    a global weight scale.  For size tests where quantizing a real input on
    the CPU would be too slow."""
    g = rng(config, 0, seed)
    ex = g.integers(127 - 10, 127 + 3, size=(B, K // 16), dtype=np.uint8).astype(np.uint32)
    mant = g.integers(0, 1 << 23, size=(B, K // 16), dtype=np.uint32)
    return {
        "a_codes": g.integers(0, 256, size=(B, K // 2), dtype=np.uint8),
        "a_scale": (np.left_shift(ex, 23) | mant).view(np.float32),
        "w_codes": g.integers(0, 256, size=(N, K // 2), dtype=np.uint8),
        "w_sf": g.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8),
        "w_g": np.array([1.0 / 2688.0], np.float32),
    }


def random_mx_operands(B: int, N: int, K: int, seed: int = SEED, config: int = 61) -> dict:
    """Arbitrary valid MXFP4 GEMM operands drawn directly in the stored formats
    (no quantization involved): uniform code bytes, E8M0 scale bytes uniform in
    [127-12, 127+3] (finite powers of two), per-row activation globals in
    [2^-4, 1) and one weight global in [2^-3, 2^-1), from uniform exponents and
    mantissa bits (outputs stay in the normal fp16 range).  For size tests where
    quantizing a real input on the CPU would be too slow."""
    g = rng(config, 0, seed)

    def pos_floats(n, lo, hi):
        ex = g.integers(127 + lo, 127 + hi, size=n, dtype=np.uint32)
        return (np.left_shift(ex, 23) | g.integers(0, 1 << 23, size=n, dtype=np.uint32)).view(np.float32)

    return {
        "a_codes": g.integers(0, 256, size=(B, K // 2), dtype=np.uint8),
        "a_sf": g.integers(127 - 12, 127 + 4, size=(B, K // 32), dtype=np.uint8),
        "a_g": pos_floats(B, -4, 0),
        "w_codes": g.integers(0, 256, size=(N, K // 2), dtype=np.uint8),
        "w_sf": g.integers(127 - 12, 127 + 4, size=(N, K // 32), dtype=np.uint8),
        "w_g": pos_floats(1, -3, -1),
    }
