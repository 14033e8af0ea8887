"""Seeded synthetic inputs, shared by the tests, the benchmark and the oracle.

Holds no step of the attention method: only random numbers. Every stream is
counter-based splitmix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", 2014): output i of a stream with seed s is the 64-bit
finaliser applied to s + (i + 1) * 0x9E3779B97F4A7C15. Uniforms take the top
24 bits (exact in binary32); normals use the Box-Muller transform in FP64;
permutations are Fisher-Yates shuffles driven by the same stream.
"""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """Outputs offset .. offset+n-1 of the stream with this seed."""
    i = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GAMMA
    return _mix(z)


def stream_seed(*tags: int) -> int:
    """Seed of the stream named by a tuple of integers (config seed, layer, tensor id, ...)."""
    s = np.uint64(0)
    for t in tags:
        s = _mix(np.array([s ^ np.uint64(t & 0xFFFFFFFFFFFFFFFF)], dtype=np.uint64))[0]
    return int(s)


def uniform(seed: int, n: int) -> np.ndarray:
    """n values in [0, 1), multiples of 2^-24 (float64)."""
    return (splitmix64(seed, n) >> np.uint64(40)).astype(np.float64) * (1.0 / (1 << 24))


def normal(seed: int, n: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """n standard normals (float64) by Box-Muller on pairs of uniforms."""
    m = (n + 1) // 2
    u = uniform(seed, 2 * m)
    u1 = 1.0 - u[0::2]  # (0, 1]
    u2 = u[1::2]
    rad = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * m)
    z[0::2] = rad * np.cos(2.0 * np.pi * u2)
    z[1::2] = rad * np.sin(2.0 * np.pi * u2)
    return mean + std * z[:n]


def permutation(seed: int, n: int) -> np.ndarray:
    """Fisher-Yates shuffle of 0..n-1 (int32)."""
    p = np.arange(n, dtype=np.int32)
    r = splitmix64(seed, max(n - 1, 0))
    for k, i in enumerate(range(n - 1, 0, -1)):
        j = int(r[k] % np.uint64(i + 1))
        p[i], p[j] = p[j], p[i]
    return p


def round_to(x: np.ndarray, dtype: str):
    """Round float64 values to the tensor dtype ('f32', 'f16', 'bf16') with
    round-to-nearest-even; returns a torch CPU tensor of that dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return t.to({"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype])


def as_f32(t) -> np.ndarray:
    """Exact binary32 widening of a torch CPU tensor (fp32/fp16/bf16) as numpy."""
    import torch
    return t.to(torch.float32).numpy()
