"""Seeded synthetic inputs shaped like the BitNet b1.58 workloads.

This module generates inputs only: it holds none of the method's arithmetic
(no quantiser, no packing, no matmul) and is shared by the tests, the smoke
check and the benchmark, so that the HIP path and the CPU oracle see the very
same bytes.  Every generator draws from ``numpy.random.default_rng(seed)`` with
seed = 1000 * workload + shape index, and rounds float32 draws to bfloat16
with round-to-nearest-even where the workload is bf16.

Workloads (model shapes from the BitNet b1.58 sources: the 2B4T model of the
asi.tokyo article, and the 3B / 70B rows of Tables 1 and 3 of the cheatsheet.md
summary "1-bit LLM era: Microsoft introduces BitNet b1.58"):

  tiny     one layer, M=4, K=256, N=512; fp32 W ~ N(0, 0.02); fp32 x ~ N(0, 1)
  decode   M=1 at 2B-class shapes (QKV, O, up/gate, down); bf16 W ~ N(0, 0.02);
           bf16 x ~ N(0, 1) with 1% of channels scaled by 20 (outliers)
  prefill  M=512 at 3B-class shapes; bf16 W ~ N(0, 0.02) with an independent
           30% of entries multiplied by 1e-3; x ~ Student-t(3) per token
  stack    30-layer 2B-class decoder, hidden 2560, FFN 6912, M=64
  xl       70B-class layer, K=8192/N=28672 and K=28672/N=8192; W ~ N(0, 0.01)
"""
from __future__ import annotations

import numpy as np

# ---- bfloat16 helpers (input representation only) ---------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the uint16 bits.
    Inputs here are finite draws, so NaN handling is not needed."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def rng_for(workload: int, shape_index: int = 0) -> np.random.Generator:
    return np.random.default_rng(1000 * workload + shape_index)


# ---- workload shapes ---------------------------------------------------------

TINY = dict(M=4, K=256, N=512)

# (name, K, N): fused QKV, attention output, fused up/gate, down (2B4T-class)
DECODE_SHAPES = [
    ("qkv", 2560, 3840),
    ("o", 2560, 2560),
    ("up_gate", 2560, 13824),
    ("down", 6912, 2560),
]

PREFILL_M = 512
PREFILL_SHAPES = [("ffn_in", 3200, 8640), ("ffn_out", 8640, 3200)]

XL_SHAPES = [("ffn_in", 8192, 28672), ("ffn_out", 28672, 8192)]
XL_MS = (1, 16, 128)

STACK = dict(layers=30, hidden=2560, heads=20, kv_heads=5, head_dim=128, ffn=6912, M=64)


# ---- generators ----------------------------------------------------------------


def tiny(seed_index: int = 0):
    """fp32 weights [N,K] and activations [M,K]."""
    rng = rng_for(1, seed_index)
    w = (rng.standard_normal((TINY["N"], TINY["K"]), dtype=np.float32) * np.float32(0.02))
    x = rng.standard_normal((TINY["M"], TINY["K"]), dtype=np.float32)
    return w, x


def normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma))


def decode_activations(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    """bf16 x ~ N(0,1) with round(0.01*K) outlier channels (same for every
    token) multiplied by 20."""
    x = rng.standard_normal((m, k), dtype=np.float32)
    n_out = int(round(0.01 * k))
    cols = rng.choice(k, size=n_out, replace=False)
    x[:, cols] *= np.float32(20.0)
    return f32_to_bf16_bits(x)


def decode(shape_index: int, m: int = 1):
    """One decode shape: (name, bf16 W bits [N,K], bf16 x bits [M,K])."""
    name, k, n = DECODE_SHAPES[shape_index]
    rng = rng_for(2, shape_index)
    w = normal_bf16(rng, (n, k), 0.02)
    x = decode_activations(rng, m, k)
    return name, w, x


def prefill(shape_index: int, m: int = PREFILL_M):
    """One prefill shape: (name, bf16 W bits, bf16 x bits)."""
    name, k, n = PREFILL_SHAPES[shape_index]
    rng = rng_for(3, shape_index)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    near_zero = rng.random((n, k)) < 0.30
    w[near_zero] *= np.float32(1e-3)
    x = rng.standard_t(3, size=(m, k)).astype(np.float32)
    return name, f32_to_bf16_bits(w), f32_to_bf16_bits(x)


def xl(shape_index: int, m: int = 1):
    """One 70B-class shape: (name, bf16 W bits, bf16 x bits)."""
    name, k, n = XL_SHAPES[shape_index]
    rng = rng_for(5, shape_index)
    w = normal_bf16(rng, (n, k), 0.01)
    x = f32_to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    return name, w, x


def stack_layer_weights(layer: int):
    """bf16 weights of one 2B-class decoder layer: dict name -> [N,K] bits.
    Seed per (layer, matrix)."""
    h, f = STACK["hidden"], STACK["ffn"]
    kv = STACK["kv_heads"] * STACK["head_dim"]
    shapes = {
        "qkv": (h + 2 * kv, h),
        "o": (h, h),
        "up_gate": (2 * f, h),
        "down": (h, f),
    }
    out = {}
    for i, (name, shp) in enumerate(shapes.items()):
        rng = np.random.default_rng(4000 + 10 * layer + i)
        out[name] = normal_bf16(rng, shp, 0.02)
    return out


def stack_input(m: int = STACK["M"]) -> np.ndarray:
    rng = rng_for(4, 999)
    return f32_to_bf16_bits(rng.standard_normal((m, STACK["hidden"]), dtype=np.float32))


def random_case(seed: int, m: int, n: int, k: int, bf16: bool = True, sigma: float = 0.02):
    """Generic seeded case for ragged and edge shapes."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(sigma)
    x = rng.standard_normal((m, k), dtype=np.float32)
    if bf16:
        return f32_to_bf16_bits(w), f32_to_bf16_bits(x)
    return w, x
