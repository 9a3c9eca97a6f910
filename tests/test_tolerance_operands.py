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


def _kernel_decode_f32(q, s, b, odd):
    """The f32 value the binary16 weight decode forms before its binary16 rounding: even nibbles
    (1024 + q)*s + (b - 1024 s), odd ones (1024 + 16 q)*(s/16) + (b - 64 s). Every product is
    exact in f32 (at most 19 significant bits), so each sum is one f32 rounding, as the fused
    multiply-adds of the kernels round."""
    f = np.float32
    if odd:
        c = (f(-64.0) * s + b).astype(f)
        return ((f(1024.0) + f(16.0) * q) * (s / f(16.0)) + c).astype(f)
    c = (f(-1024.0) * s + b).astype(f)
    return ((f(1024.0) + q) * s + c).astype(f)


def _bf16_draw(rng, n, lo_exp, hi_exp):
    """n bf16 values, random sign, 8-bit significand, binary exponent uniform in [lo_exp, hi_exp)."""
    sig = 1.0 + rng.integers(0, 128, n) / 128.0
    return _bf16(np.where(rng.random(n) < 0.5, -1.0, 1.0) * sig * np.exp2(rng.integers(lo_exp, hi_exp, n)))


def test_weight_decode_is_single_rounding_inside_the_band():
    """For |b| in [2^-6, 2^15) |s|, and for b = 0, the decode's f32 value is q*s + b exactly, so the
    binary16 weight is q*s + b rounded once: equal to float64 -> binary16 on both nibble paths
    wherever q*s + b is a finite binary16 value. The one difference in bits is the sign of a zero
    weight (q = 0 with b = -0 gives +0, not -0), which no product sum can see."""
    rng = np.random.default_rng(77)
    n = 200_000
    s = _bf16_draw(rng, n, -12, 3)
    ratio = np.exp2(rng.integers(-6, 15, n)) * (1.0 + rng.integers(0, 128, n) / 128.0)
    b = _bf16(np.where(rng.random(n) < 0.5, -1.0, 1.0) * np.abs(s) * ratio)
    b[: n // 10] = 0.0                                     # bias 0
    q = rng.integers(0, 16, n).astype(np.float32)
    z = rng.integers(0, 16, n // 10)                       # bias -zero_point * scale, zero point 0..15
    b[n // 10: n // 5] = _bf16(-z * s[n // 10: n // 5].astype(np.float64))
    exact = q.astype(np.float64) * s.astype(np.float64) + b.astype(np.float64)
    fits = np.abs(exact) < 65504.0
    assert fits.mean() > 0.9
    for odd in (False, True):
        v = _kernel_decode_f32(q, s, b, odd)
        assert np.array_equal(v.astype(np.float64), exact), f"odd={odd}: f32 value not exact"
        assert np.array_equal(v[fits].astype(np.float16), exact[fits].astype(np.float16)), f"odd={odd}"


@pytest.mark.parametrize("side", ["below", "above"])
def test_weight_decode_error_outside_the_band_is_bounded(side):
    """Outside the band the f32 step can round before the binary16 rounding. Below it (|b| down to
    2^-40 |s|) the error is at most 2^-14 |s|; above it (|b| up to 2^40 |s|) at most 2^-22 |b|, a
    relative error at f32's scale. Both bounds hold, and just past each band edge the rounding
    does happen, so the band is not wider than stated by more than a factor of two."""
    rng = np.random.default_rng(78 if side == "below" else 79)
    n = 200_000
    s = _bf16_draw(rng, n, -40, 3)
    lo, hi, edge = (-40, -6, (-8, -6)) if side == "below" else (16, 40, (16, 18))
    ratio_exp = rng.integers(lo, hi, n)
    ratio_exp[: n // 4] = rng.integers(*edge, n // 4)      # a quarter just past the edge
    ratio = np.exp2(ratio_exp) * (1.0 + rng.integers(0, 128, n) / 128.0)
    b = _bf16(np.where(rng.random(n) < 0.5, -1.0, 1.0) * np.abs(s) * ratio)
    q = rng.integers(0, 16, n).astype(np.float32)
    exact = q.astype(np.float64) * s.astype(np.float64) + b.astype(np.float64)
    bound = np.abs(s.astype(np.float64)) * 2.0 ** -14 if side == "below" else np.abs(b.astype(np.float64)) * 2.0 ** -22
    for odd in (False, True):
        err = np.abs(_kernel_decode_f32(q, s, b, odd).astype(np.float64) - exact)
        assert (err <= bound).all(), f"odd={odd}"
        if not (odd and side == "below"):                  # the odd path's lower edge sits lower
            assert (err[: n // 4] > 0).any(), f"odd={odd}: no rounding just past the edge"
