"""Seeded synthetic inputs for the three 4-bit weight encodings.

This module only draws random numbers and stores them in the operand layouts;
it holds none of the dequantize-and-multiply arithmetic. Both the HIP path and
the CPU oracle are fed from here.

Distributions (one numpy PCG64 stream per call, draws in the order written):

* affine INT4, group 32 (INT4 MatMulNBits page): packed words uint32 [N, K/8]
  uniform over all 32-bit values, which is the same as eight independent
  uniform nibbles 0..15 per word; zero-points uniform integers 0..15; scales
  uniform [0.005, 0.02) rounded to bf16; bias = bf16(-zp * scale) taken from the
  unrounded f32 scale, as the page's test builds it; x ~ N(0, 1) rounded to bf16.
* lookup codebook (lut4 page): packed index bytes uniform 0..255 (two uniform
  codes per byte); per-block scales uniform [0.01, 0.05) rounded to fp16,
  block 64 along the flat index; x ~ N(0, 1) rounded to fp16; the frozen
  codebook is the 16 sorted standard-normal quantiles at (i + 0.5) / 16,
  rounded to f32.
* expert-routed GGML Q4_0 (mlx-native MoE page): per block a scale d uniform
  [0.002, 0.01) rounded to fp16 and 16 uniform bytes of nibble pairs; blocks
  stored as 18 bytes (little-endian d, then the 16 bytes); x ~ N(0, 1) f32;
  per token top_k distinct expert ids drawn uniformly without replacement.
"""
from __future__ import annotations

import numpy as np
import torch

Q4_0_QK = 32
Q4_0_BYTES = 18


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def affine_case(M: int, K: int, N: int, seed: int = 0, group: int = 32,
                scale_range=(0.005, 0.02), x_scale: float = 1.0):
    rng = np.random.default_rng(seed)
    w = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    zp = rng.integers(0, 16, size=(N, K // group)).astype(np.float32)
    s = rng.uniform(scale_range[0], scale_range[1], size=(N, K // group)).astype(np.float32)
    x = (rng.standard_normal((M, K)) * x_scale).astype(np.float32)
    return {
        "w": w,
        "scales": _to_bf16_bits(s),
        "biases": _to_bf16_bits(-zp * s),
        "x": _to_bf16_bits(x),
        "M": M, "K": K, "N": N, "group": group,
    }


def normal_codebook() -> np.ndarray:
    from scipy.stats import norm
    return norm.ppf((np.arange(16) + 0.5) / 16.0).astype(np.float32)


def lut_case(M: int, K: int, N: int, seed: int = 0, block: int = 64,
             scale_range=(0.01, 0.05)):
    rng = np.random.default_rng(seed)
    count = N * K
    blocks = -(-count // block)
    packed = rng.integers(0, 256, size=blocks * block // 2, dtype=np.uint16).astype(np.uint8)
    scales = rng.uniform(scale_range[0], scale_range[1], size=blocks).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    return {
        "packed": packed,
        "scales": _to_f16_bits(scales),
        "book": normal_codebook(),
        "x": _to_f16_bits(x),
        "M": M, "K": K, "N": N, "block": block,
    }


def q4_0_blocks(rng, shape_rows, K: int, d_range=(0.002, 0.01)):
    """GGML Q4_0 rows: bytes [*shape_rows, (K/32)*18]."""
    nb = K // Q4_0_QK
    d = rng.uniform(d_range[0], d_range[1], size=tuple(shape_rows) + (nb,)).astype(np.float32)
    qs = rng.integers(0, 256, size=tuple(shape_rows) + (nb, 16), dtype=np.uint16).astype(np.uint8)
    blk = np.empty(tuple(shape_rows) + (nb, Q4_0_BYTES), np.uint8)
    blk[..., 0:2] = _to_f16_bits(d).astype("<u2").view(np.uint8).reshape(d.shape + (2,))
    blk[..., 2:] = qs
    return blk.reshape(tuple(shape_rows) + (nb * Q4_0_BYTES,))


def moe_case(n_experts: int, N: int, K: int, n_tokens: int, top_k: int, seed: int = 0,
             d_range=(0.002, 0.01)):
    rng = np.random.default_rng(seed)
    w = q4_0_blocks(rng, (n_experts, N), K, d_range)
    x = rng.standard_normal((n_tokens, K)).astype(np.float32)
    ids = np.stack([rng.choice(n_experts, size=top_k, replace=False) for _ in range(n_tokens)])
    ids = ids.astype(np.uint32).reshape(-1)
    row_bytes = (K // Q4_0_QK) * Q4_0_BYTES
    return {
        "w": w.reshape(-1),
        "x": x,
        "ids": ids,
        "n_experts": n_experts, "N": N, "K": K, "n_tokens": n_tokens, "top_k": top_k,
        "expert_stride": N * row_bytes,
    }


def moe_swiglu_case(n_experts: int, N: int, K: int, n_tokens: int, top_k: int, seed: int = 0,
                    d_range=(0.002, 0.01)):
    """moe_case's weights and ids, plus per-routed-row gate and up, f32 ~ N(0, 1) each
    (drawn from their own generator, seed + 1, gate first)."""
    c = moe_case(n_experts, N, K, n_tokens, top_k, seed, d_range)
    rng = np.random.default_rng(seed + 1)
    rows = n_tokens * top_k
    c["gate"] = rng.standard_normal((rows, K)).astype(np.float32)
    c["up"] = rng.standard_normal((rows, K)).astype(np.float32)
    return c


# The workloads the path is measured and checked on.
def tiny_affine(seed: int = 0):
    return affine_case(4, 256, 256, seed)


def decode_affine(seed: int = 0):
    return affine_case(1, 4096, 14336, seed)


def prefill_affine(seed: int = 0):
    return affine_case(2048, 4096, 4096, seed)


def lut_matmul_case(seed: int = 0):
    return lut_case(512, 4096, 11008, seed)


def moe_q4_0_case(seed: int = 0):
    return moe_case(64, 1408, 2048, 128, 8, seed)


def moe_swiglu_decode_case(seed: int = 0):
    """One decode token through the fused SwiGLU routed mat-vec, on the MoE workload's experts."""
    return moe_swiglu_case(64, 1408, 2048, 1, 8, seed)
