"""The affine matrix-core arithmetic stays inside the stated bound (CPU only).

The bound |y - ref| <= 1e-2 |ref| + 1e-2 sqrt(K) max|x| max|scale| is tightest
at small K, where few products make up |ref|. These tests emulate, in numpy,
the operands the affine matrix-core kernels multiply (x converted bf16 ->
binary16, each weight q*s + b formed in f32 and rounded once to binary16,
products accumulated in f32, bf16 output) and check that every output of
many seeded shapes, the short-K cases included, lies inside the bound
against the oracle. They also record why the operands are binary16 and not
bf16: with the weights rounded to bf16 (8 significant bits) one output of the
random-shape case with seed 4 (M=47, K=64, N=128) falls outside the bound.
"""
import numpy as np
import pytest
import torch

import oracle
from weight_only_bit_w4_amd import synth


def _bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _f16(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, np.float32).astype(np.float16).astype(np.float32)


def _emulated(c, operand) -> np.ndarray:
    """y as the kernels form it with the given operand rounding (binary16 or bf16)."""
    M, K, N = c["M"], c["K"], c["N"]
    s = oracle.bf16_to_f32(c["scales"])
    b = oracle.bf16_to_f32(c["biases"])
    x = oracle.bf16_to_f32(c["x"])
    q = np.zeros((N, K), np.float32)
    for j in range(8):
        q[:, j::8] = ((c["w"] >> (4 * j)) & 15).astype(np.float32)
    g = np.repeat(np.arange(K // 32), 32)
    w = (q * s[:, g] + b[:, g]).astype(np.float32)          # q*s exact, one f32 rounding for + b
    acc = operand(x).astype(np.float32) @ operand(w).astype(np.float32).T   # f32 accumulation
    return _bf16(acc).astype(np.float64)


def _outside(c, operand) -> int:
    M, K, N = c["M"], c["K"], c["N"]
    ref, _ = oracle.affine(c["w"], c["scales"], c["biases"], c["x"], M, K, N)
    ms = float(np.abs(oracle.bf16_to_f32(c["scales"])).max())
    mx = float(np.abs(oracle.bf16_to_f32(c["x"])).max())
    return int((np.abs(_emulated(c, operand) - ref) > oracle.tolerance(ref, K, mx, ms)).sum())


def _sweep_shape(seed):
    # the random-shape GPU sweep's affine shapes (tests/test_parity_gpu_sweep.py)
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.choice([1, 2, 3, 5, 6, 9, 16, 23, 32, 47, 64, 65, 80]))
    K = 64 * int(rng.integers(1, 41))
    N = 32 * int(rng.integers(1, 33))
    return M, K, N


@pytest.mark.parametrize("seed", range(40))
def test_binary16_operands_stay_inside_on_random_shapes(seed):
    M, K, N = _sweep_shape(seed)
    assert _outside(synth.affine_case(M, K, N, seed=seed), _f16) == 0


@pytest.mark.parametrize("K", [32, 64, 96, 128])
@pytest.mark.parametrize("seed", range(6))
def test_binary16_operands_stay_inside_at_short_k(K, seed):
    assert _outside(synth.affine_case(64, K, 512, seed=100 * K + seed), _f16) == 0


def test_bf16_operands_would_exceed_the_bound_at_one_output():
    c = synth.affine_case(47, 64, 128, seed=4)
    assert _outside(c, _bf16) == 1
    assert _outside(c, _f16) == 0
