"""Seeded synthetic inputs and the workload table.

This module holds no quantization arithmetic: it draws random tensors with
numpy's PCG64 generator and rounds them to bf16 (round-to-nearest-even,
torch's CPU cast). Both the GPU library's tests and the oracle's tests take
their inputs from here, so both sides see identical bytes.

The shapes follow transformer linears: 8192 tokens, hidden 4096 and FFN
14336 (the Megatron Llama-like configuration on the page "从 BF16 到
FP8/FP4", section 4.2), and DeepSeek-V3-like 7168 x 18432 weights. The
distributions are normal activations, small-variance normal gradients and
weights, and heavy-tailed Student-t values for MX blocks.

bf16 tensors are handled as numpy uint16 arrays of their bit patterns.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

BF16 = "bf16"
F32 = "f32"


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, rounded to nearest even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> fp32 values (exact widening)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(shape, std: float, seed: int, dtype: str = BF16) -> np.ndarray:
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    x = rng.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    x = x.reshape(shape)
    return to_bf16_bits(x) if dtype == BF16 else x


def student_t(shape, nu: float, seed: int, dtype: str = BF16) -> np.ndarray:
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    x = rng.standard_t(nu, size=n).astype(np.float32).reshape(shape)
    return to_bf16_bits(x) if dtype == BF16 else x


def normal_with_outliers(n: int, seed: int, outlier_seed: int, count: int = 64,
                         magnitude: float = 1000.0) -> np.ndarray:
    """fp32 N(0,1) with `count` entries replaced by +-magnitude at random
    positions and signs, so the tensor amax is exactly `magnitude`."""
    x = np.random.default_rng(seed).standard_normal(n, dtype=np.float32)
    rng = np.random.default_rng(outlier_seed)
    pos = rng.permutation(n)[:count]
    sign = rng.integers(0, 2, size=count)
    x[pos] = np.where(sign == 1, np.float32(magnitude), np.float32(-magnitude))
    return x


def uniform_bits_bf16(shape, seed: int, max_abs: float = 1e4) -> np.ndarray:
    """bf16 values spread over many binades: sign * 2^U(-40, log2 max_abs)."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    e = rng.uniform(-40.0, np.log2(max_abs), size=n)
    s = rng.choice([-1.0, 1.0], size=n)
    return to_bf16_bits((s * np.exp2(e)).astype(np.float32).reshape(shape))


@dataclass
class Workload:
    """One tensor to quantize: name, shape, input dtype, generator, recipe."""
    name: str
    shape: Tuple[int, int]
    dtype: str
    recipe: str            # "current" | "delayed" | "block" | "mx" | "nvfp4"
    fmt: str = "e4m3"      # "e4m3" | "e5m2" | "e2m1"
    block: Optional[Tuple[int, int]] = None
    outputs: int = 1       # 1 rowwise, 2 colwise, 3 both
    seed: int = 0
    dist: str = "normal"   # "normal" | "student_t" | "outliers"
    std: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def numel(self) -> int:
        return self.shape[0] * self.shape[1]

    def make(self, seed: Optional[int] = None) -> np.ndarray:
        s = self.seed if seed is None else seed
        if self.dist == "normal":
            return normal(self.shape, self.std, s, self.dtype)
        if self.dist == "student_t":
            return student_t(self.shape, self.extra.get("nu", 3.0), s, self.dtype)
        if self.dist == "outliers":
            x = normal_with_outliers(self.numel, s, self.extra["outlier_seed"])
            return x.reshape(self.shape)
        raise ValueError(self.dist)


# The benchmark and full-size parity workloads.
SMALL_CURRENT = Workload("current_e4m3_f32_1m", (1, 1 << 20), F32, "current", "e4m3", seed=1001,
                         dist="outliers", extra={"outlier_seed": 1002})

LARGE = [
    Workload("current_e4m3_act_8192x4096", (8192, 4096), BF16, "current", "e4m3", seed=2001),
    Workload("current_e5m2_grad_8192x4096", (8192, 4096), BF16, "current", "e5m2", seed=2002, std=1e-3),
    Workload("delayed_e4m3_act_8192x4096", (8192, 4096), BF16, "delayed", "e4m3", seed=2100,
             extra={"history_len": 1024}),
    Workload("delayed_e5m2_grad_8192x4096", (8192, 4096), BF16, "delayed", "e5m2", seed=2200, std=1e-3,
             extra={"history_len": 1024}),
    Workload("block1x128_act_16384x7168", (16384, 7168), BF16, "block", "e4m3", block=(1, 128), seed=3001),
    Workload("block128x128_wgt_7168x18432", (7168, 18432), BF16, "block", "e4m3", block=(128, 128), seed=3002,
             std=0.02),
    Workload("mxfp8_rowcol_8192x8192", (8192, 8192), BF16, "mx", "e4m3", block=(1, 32), outputs=3, seed=4001,
             dist="student_t", extra={"nu": 3.0}),
    Workload("nvfp4_1x16_act_8192x14336", (8192, 14336), BF16, "nvfp4", "e2m1", block=(1, 16), seed=5001),
    Workload("nvfp4_16x16_wgt_14336x4096", (14336, 4096), BF16, "nvfp4", "e2m1", block=(16, 16), seed=5002,
             std=0.02),
]

BY_NAME = {w.name: w for w in [SMALL_CURRENT, *LARGE]}
