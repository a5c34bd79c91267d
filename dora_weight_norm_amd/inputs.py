"""Seeded synthetic inputs for the DoRA norm and compose.

This module only draws random numbers and rounds them to the storage type;
it holds none of the method's arithmetic. Both the HIP path (tests, bench)
and the CPU oracle consume what it returns, so it imports nothing from
either.

Each tensor comes from its own PCG64 stream, ``SeedSequence(seed,
spawn_key=(k,))`` with a fixed k per tensor, so drawing one tensor never
shifts another. Values are drawn in fp64, rounded to fp32 (RNE), and for
bf16 workloads rounded once more to bf16 (RNE); the returned float32 arrays
hold exactly those storage values.

Distributions (the workload shapes and g statistics come from the DoRA
write-ups: d_in = 8192 at r = 384, the 8192 x 28672 MLP shape, KV d_out =
512, ranks up to 768, and magnitude scales g near 1 with spread 0.0015):
    W     ~ N(0, 1/d_in)        A    ~ N(0, 1/d_in)       B ~ N(0, 0.02^2)
    base  ~ N(0, 1)             lora ~ N(0, 0.1^2)
    m_noise ~ N(0, 1)   (the magnitude is m = wnorm * (1 + 0.0015 m_noise);
                         the product with wnorm is left to the caller)
    dy    ~ N(0, 1)             an upstream gradient for the compose backward
    g     = fp32(1 + 0.0015 N(0, 1))  for compose-only runs
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "HEADLINE",
    "STREAMS",
    "normal",
    "to_storage",
    "norm_inputs",
    "compose_inputs",
    "m_noise",
    "grad_inputs",
    "activations",
]

MiB = 1 << 20

# Stream ids, one per tensor.
STREAMS = {"W": 0, "A": 1, "B": 2, "m_noise": 3, "base": 4, "lora": 5, "g": 6, "dy": 7, "wnorm": 8, "x": 9}

G_SPREAD = 0.0015      # std of the magnitude scale g around 1
B_STD = 0.02
LORA_STD = 0.1


@dataclass(frozen=True)
class Workload:
    name: str
    d_out: int
    d_in: int
    r: int
    s: float
    dtype: str          # "bf16" or "f32"
    T: int              # compose rows (batch x seq)
    seed: int
    budget: int = 256 * MiB
    eps: float = 1e-6


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32_256x256_r8", 256, 256, 8, 2.0, "f32", 64, 0),
        Workload("qproj_4096x4096_r64", 4096, 4096, 64, 2.0, "bf16", 4096, 1),
        Workload("headline_8192x8192_r384", 8192, 8192, 384, 0.5, "bf16", 8192, 2),
        Workload("mlp_28672x8192_r512", 28672, 8192, 512, 0.5, "bf16", 8192, 3),
        Workload("kv_512x3584_r768", 512, 3584, 768, 0.25, "bf16", 8192, 40),
        Workload("square_8192x8192_r768", 8192, 8192, 768, 0.25, "bf16", 16384, 41),
    ]
}
HEADLINE = WORKLOADS["headline_8192x8192_r384"]


def _rng(seed: int, stream: str) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(STREAMS[stream],))
    return np.random.Generator(np.random.PCG64(ss))


def normal(seed: int, stream: str, shape, std: float = 1.0, mean: float = 0.0):
    """fp64 draws from N(mean, std^2) on the tensor's own stream."""
    x = _rng(seed, stream).standard_normal(shape)
    if std != 1.0:
        x *= std
    if mean != 0.0:
        x += mean
    return x


def _f32_to_bf16_values(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (RNE on the upper 16 bits); returns float32 values."""
    u = x32.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    hi = (u + bias) & np.uint32(0xFFFF0000)
    return hi.view(np.float32)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 or fp16 (RNE) for those dtypes; float32 result."""
    x32 = np.ascontiguousarray(x64, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return _f32_to_bf16_values(x32)
    if dtype == "f16":
        return x32.astype(np.float16).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def norm_inputs(d_out: int, d_in: int, r: int, dtype: str, seed: int):
    """W [d_out, d_in], A [r, d_in], B [d_out, r] as float32 storage values."""
    sd = 1.0 / np.sqrt(d_in) if d_in > 0 else 1.0
    W = to_storage(normal(seed, "W", (d_out, d_in), sd), dtype)
    A = to_storage(normal(seed, "A", (r, d_in), sd), dtype)
    B = to_storage(normal(seed, "B", (d_out, r), B_STD), dtype)
    return W, A, B


def m_noise(d_out: int, seed: int) -> np.ndarray:
    """N(0,1) draws for the magnitude perturbation, fp64."""
    return normal(seed, "m_noise", (d_out,))


def compose_inputs(T: int, d_out: int, dtype: str, seed: int):
    """base, lora [T, d_out] as storage values; g [d_out] fp32 near 1."""
    base = to_storage(normal(seed, "base", (T, d_out)), dtype)
    lora = to_storage(normal(seed, "lora", (T, d_out), LORA_STD), dtype)
    g = normal(seed, "g", (d_out,), G_SPREAD, 1.0).astype(np.float32)
    return base, lora, g


def grad_inputs(T: int, d_out: int, dtype: str, seed: int):
    """dy [T, d_out] (storage values) for the compose backward, plus a
    positive fp32 stand-in row norm wnorm = 1 + |N(0,1)| for dm."""
    dy = to_storage(normal(seed, "dy", (T, d_out)), dtype)
    wnorm = (1.0 + np.abs(normal(seed, "wnorm", (d_out,)))).astype(np.float32)
    return dy, wnorm


def activations(T: int, d_in: int, dtype: str, seed: int):
    """Layer input x [T, d_in] ~ N(0, 1) (storage values), for the whole
    DoRA linear layer."""
    return to_storage(normal(seed, "x", (T, d_in)), dtype)
