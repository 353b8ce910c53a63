"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no quantization arithmetic: it only draws random tensors of
the shapes and distributions the pages study and rounds them to the storage
dtype.  Real model tensors (the Llama / Qwen / Granite dumps the pages measure
on) are not available; these stand in for them.

Arrays are numpy: fp32 as ``float32``, bf16 as raw ``uint16`` bits.

Workloads (shapes follow Llama-8B-style linear layers: hidden 4096, MLP 14336):
  w1  fp32 1024x1024 ~ N(0, 0.02^2)                         (seed 101)
  w2  bf16 8192x4096 ~ N(0, sigma^2), sigma in {1e-3, 2e-2}  (seed 102)
  w3  bf16 4096x14336 ~ Laplace(0, 1e-4), 0.1% entries x50    (seed 103)
  w4  bf16 16384x4096 ~ Laplace(0, 1), 8 columns x100         (seed 104)
  w5  bf16 A 8192x4096 ~ N(0, 1) (seed 105), B 14336x4096 ~ N(0, 0.02^2) (seed 205)
Every generator takes the shape, so the tests can draw the same distribution
at small sizes.
"""
import numpy as np

SR_SEED = 0x00C0FFEE12345678


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x):
    """Nearest bf16 (ties to even) of finite fp32 values, as uint16 bits."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    return (r >> 16).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(shape, sigma, seed, dtype="bf16"):
    x = _rng(seed).standard_normal(shape, dtype=np.float32)
    x *= np.float32(sigma)
    return to_bf16_bits(x) if dtype == "bf16" else x


def laplace(shape, b, seed):
    rng = _rng(seed)
    x = rng.standard_exponential(shape, dtype=np.float32)
    sign = rng.integers(0, 2, shape, dtype=np.int8)
    x[sign == 1] *= -1
    x *= np.float32(b)
    return x, rng


def w1(shape=(1024, 1024), seed=101):
    return normal(shape, 0.02, seed, dtype="f32")


def w2(sigma, shape=(8192, 4096), seed=102):
    return normal(shape, sigma, seed)


def w3(shape=(4096, 14336), seed=103, frac=0.001, boost=50.0):
    x, rng = laplace(shape, 1e-4, seed)
    n = x.size
    k = max(1, int(round(frac * n)))
    idx = rng.choice(n, size=k, replace=False)
    x.reshape(-1)[idx] *= np.float32(boost)
    return to_bf16_bits(x)


def w4(shape=(16384, 4096), seed=104, channels=8, boost=100.0):
    x, rng = laplace(shape, 1.0, seed)
    cols = rng.choice(shape[1], size=min(channels, shape[1]), replace=False)
    x[:, cols] *= np.float32(boost)
    return to_bf16_bits(x)


def w5(m=8192, n=14336, k=4096, seed_a=105, seed_b=205):
    a = normal((m, k), 1.0, seed_a)
    b = normal((n, k), 0.02, seed_b)
    return a, b
