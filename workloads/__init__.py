"""Seeded synthetic inputs for the BitLinear forward, shared by both sides of every check.

This module only *draws* tensors: Gaussian fp32 weights, ternary code matrices with a given
code mix, Gaussian activations (optionally with outlier channels, optionally rounded to bf16)
and RMSNorm weights.  It holds none of the method's arithmetic (no scale reduction, no
quantization, no packing, no product), so the CPU oracle and the GPU path can both take their
inputs from here without sharing any computation.

Shapes and statistics follow the pages' models:

* Distillix README, "Architecture" block: hidden 768, 12 query / 4 KV heads of dim 64,
  MLP hidden 2048.
* SLM750-Edge 1.58-bit model card, §2.2 "Layer Configuration": hidden 1536, FFN 4096 (ReLU²),
  12 query / 4 KV heads, head dim 128.
* Distillix 125M model card, weight-statistics table: code mix 29 % / 42 % / 29 % and a
  weight scale of about 0.021.
* BitDistill article (Qwen3 0.6B / 1.7B / 4B students): SubLN before the attention output
  projection and before the FFN output projection.

Stream layout: every tensor comes from its own ``numpy.random.Generator(PCG64)`` seeded with
``[seed, config, matrix, role, M]`` (``M`` = 0 for tensors that do not depend on the token
count).  Roles: 0 = W, 1 = X, 2 = outlier channel indices, 3 = RMSNorm weight g,
4 = ternary codes.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Tuple

import numpy as np

ROLE_W, ROLE_X, ROLE_OUTLIER, ROLE_G, ROLE_CODES = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Matrix:
    """One BitLinear projection: ``N`` output features, ``K`` input features.

    ``norm`` marks projections whose input passes through the SubLN RMSNorm first
    (attention output projection and FFN down projection)."""

    name: str
    N: int
    K: int
    norm: bool = False


@dataclass(frozen=True)
class Workload:
    """A named set of BitLinear projections run at one or more token counts."""

    key: str
    index: int
    description: str
    matrices: Tuple[Matrix, ...]
    token_counts: Tuple[int, ...]
    weights: str  # "fp32": Gaussian fp32 master weights; "codes": pre-ternarized codes + gamma
    x_dtype: str  # "f32" or "bf16"
    w_sigma: float = 0.02
    code_mix: Tuple[float, float, float] = (0.29, 0.42, 0.29)  # P(-1), P(0), P(+1)
    code_gamma: float = 0.021
    outlier_frac: float = 0.0
    outlier_gain: float = 20.0
    decode_prepacked: bool = True  # token counts <= 16 use weights packed once, outside timing
    ffn: str = "swiglu"  # FFN activation of the layer the set belongs to: swiglu or relu2 (ungated)


WORKLOADS = {
    "c1_single_768x2048": Workload(
        key="c1_single_768x2048", index=0,
        description="single BitLinear 768->2048 (Distillix MLP up projection), 16 tokens",
        matrices=(Matrix("up", 2048, 768),),
        token_counts=(16,), weights="fp32", x_dtype="f32", decode_prepacked=False),
    "c2_distillix125m_layer": Workload(
        key="c2_distillix125m_layer", index=1,
        description="Distillix-125M layer BitLinear set: decode (1 token) and prefill (2048 tokens)",
        matrices=(Matrix("q", 768, 768), Matrix("k", 256, 768), Matrix("v", 256, 768),
                  Matrix("o", 768, 768), Matrix("gate", 2048, 768), Matrix("up", 2048, 768),
                  Matrix("down", 768, 2048)),
        token_counts=(1, 2048), weights="fp32", x_dtype="f32"),
    "c3_edge1p4b_prepacked": Workload(
        key="c3_edge1p4b_prepacked", index=2,
        description="1.4B edge shape with pre-ternarized packed weights, 1 / 8 / 512 tokens",
        matrices=(Matrix("up", 4096, 1536), Matrix("down", 1536, 4096),
                  Matrix("qkv", 2560, 1536), Matrix("o", 1536, 1536)),
        token_counts=(1, 8, 512), weights="codes", x_dtype="f32", outlier_frac=0.01,
        ffn="relu2"),
    "c4_qwen3_1p7b_subln": Workload(
        key="c4_qwen3_1p7b_subln", index=3,
        description="Qwen3-1.7B-shaped SubLN block, 4096 tokens, bf16 activations",
        matrices=(Matrix("o", 2048, 2048, norm=True), Matrix("down", 2048, 6144, norm=True),
                  Matrix("gate", 6144, 2048), Matrix("up", 6144, 2048)),
        token_counts=(4096,), weights="fp32", x_dtype="bf16", decode_prepacked=False),
    "c5_qwen3_4b_layer": Workload(
        key="c5_qwen3_4b_layer", index=4,
        description="Qwen3-4B-shaped layer set: 1-token decode on pre-packed weights and an "
                    "8192-token training-style forward that re-quantizes fp32 master weights",
        matrices=(Matrix("q", 4096, 2560), Matrix("k", 1024, 2560), Matrix("v", 1024, 2560),
                  Matrix("o", 2560, 4096), Matrix("gate", 9728, 2560), Matrix("up", 9728, 2560),
                  Matrix("down", 2560, 9728)),
        token_counts=(1, 8192), weights="fp32", x_dtype="f32"),
}


def by_index(i: int) -> Workload:
    for w in WORKLOADS.values():
        if w.index == i:
            return w
    raise KeyError(i)


def _rng(seed: int, wl: Workload, mat: int, role: int, M: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, wl.index, mat, role, M]))


def weight_fp32(wl: Workload, mat: int, seed: int = 0) -> np.ndarray:
    """Gaussian fp32 master weights [N, K] ~ N(0, sigma^2), row-major (out, in)."""
    m = wl.matrices[mat]
    z = _rng(seed, wl, mat, ROLE_W).standard_normal((m.N, m.K), dtype=np.float32)
    return z * np.float32(wl.w_sigma)


def weight_codes(wl: Workload, mat: int, seed: int = 0) -> np.ndarray:
    """I.i.d. ternary codes [N, K] int8 in {-1, 0, +1} drawn with the workload's code mix."""
    m = wl.matrices[mat]
    g = _rng(seed, wl, mat, ROLE_CODES)
    return g.choice(np.array([-1, 0, 1], dtype=np.int8), size=(m.N, m.K), p=list(wl.code_mix))


def activations_f32(wl: Workload, mat: int, M: int, seed: int = 0) -> np.ndarray:
    """Activations [M, K] fp32 ~ N(0, 1); when the workload has outlier channels, round(frac*K)
    channels chosen without replacement are multiplied by the outlier gain."""
    m = wl.matrices[mat]
    x = _rng(seed, wl, mat, ROLE_X, M).standard_normal((M, m.K), dtype=np.float32)
    if wl.outlier_frac > 0:
        n_out = int(round(wl.outlier_frac * m.K))
        ch = _rng(seed, wl, mat, ROLE_OUTLIER).choice(m.K, size=n_out, replace=False)
        x[:, ch] *= np.float32(wl.outlier_gain)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even) and return the raw uint16 bits.
    Input preparation only: NaN is not expected in synthetic data."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def activations(wl: Workload, mat: int, M: int, seed: int = 0) -> np.ndarray:
    """Activations in the workload's dtype: fp32 array, or bf16 as raw uint16 bits."""
    x = activations_f32(wl, mat, M, seed)
    return f32_to_bf16_bits(x) if wl.x_dtype == "bf16" else x


def norm_weight(wl: Workload, mat: int, seed: int = 0, kind: str = "ones") -> np.ndarray:
    """RMSNorm weight g [K]: all ones (benchmarks) or 1 + 0.1 * N(0, 1) (parity tests)."""
    K = wl.matrices[mat].K
    if kind == "ones":
        return np.ones(K, dtype=np.float32)
    z = _rng(seed, wl, mat, ROLE_G).standard_normal(K, dtype=np.float32)
    return np.float32(1.0) + np.float32(0.1) * z


def gaussian(shape, seed_key, scale: float = 1.0) -> np.ndarray:
    """Generic seeded fp32 Gaussian for ad-hoc test shapes (ragged sizes, edge cases)."""
    g = np.random.Generator(np.random.PCG64(list(seed_key)))
    return g.standard_normal(shape, dtype=np.float32) * np.float32(scale)


def ternary(shape, seed_key, mix=(0.29, 0.42, 0.29)) -> np.ndarray:
    """Generic seeded ternary code matrix for ad-hoc test shapes."""
    g = np.random.Generator(np.random.PCG64(list(seed_key)))
    return g.choice(np.array([-1, 0, 1], dtype=np.int8), size=shape, p=list(mix))
