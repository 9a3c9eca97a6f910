"""Seeded random-shape parity sweep over every entry point against the oracle.

Each case draws its shape from its own seed (printed in the failure message),
so the sweep crosses the routes inside each entry point (GEMV, shared-x and
weight-tile forms, the prefill tiles, both lookup layouts and their aligned
and element-wise forms, the MoE mat-vec and grouped GEMM) at sizes the oracle
finishes in well under a second each.
"""
import numpy as np
import pytest
import torch

import oracle
from weight_only_bit_w4_amd import binding as B
from weight_only_bit_w4_amd import synth
from test_parity_gpu import (_affine_dev, _affine_scales, _assert_within, _bf16_to_f64, _lut_dev, _lut_f32_case,
                             _max_d, _moe_run, _t)

pytestmark = pytest.mark.gpu

SEEDS = range(12)


def _affine_shape(seed):
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.choice([1, 2, 3, 5, 6, 9, 16, 23, 32, 47, 64, 65, 80]))
    K = 64 * int(rng.integers(1, 41))            # 64 .. 2560
    N = 32 * int(rng.integers(1, 33))            # 32 .. 1024
    return M, K, N


@pytest.mark.parametrize("seed", SEEDS)
def test_sweep_affine(seed):
    M, K, N = _affine_shape(seed)
    c = synth.affine_case(M, K, N, seed=seed)
    w, s, b, x = _affine_dev(c)
    y = (B.qmv_affine4 if M == 1 else B.qmm_affine4)(w, s, b, x)
    torch.cuda.synchronize()
    acc, _ = oracle.affine(c["w"], c["scales"], c["biases"], c["x"], M, K, N)
    ms, mx = _affine_scales(c)
    _assert_within(_bf16_to_f64(y), acc, K, mx, ms, f"sweep affine seed={seed} M={M} K={K} N={N}")


def _prefill_shape(seed):
    # The matrix-core prefill tiles (M > 64, K % 64 == 0), half of them with K % 256 == 0 (scales and
    # biases loaded four steps at a time), several row and column tiles, ragged edges.
    rng = np.random.default_rng(1500 + seed)
    M = int(rng.integers(65, 700))
    K = (256 if seed % 2 == 0 else 64) * int(rng.integers(1, 11))
    N = 32 * int(rng.integers(1, 25))
    return M, K, N


@pytest.mark.parametrize("seed", range(8))
def test_sweep_prefill(seed):
    M, K, N = _prefill_shape(seed)
    c = synth.affine_case(M, K, N, seed=100 + seed)
    w, s, b, x = _affine_dev(c)
    y = B.qmm_affine4(w, s, b, x)
    torch.cuda.synchronize()
    acc, _ = oracle.affine(c["w"], c["scales"], c["biases"], c["x"], M, K, N)
    ms, mx = _affine_scales(c)
    _assert_within(_bf16_to_f64(y), acc, K, mx, ms, f"sweep prefill seed={seed} M={M} K={K} N={N}")


def _tiles_shape(seed):
    # The weight-tile form (K % 256 == 0, rows past one pass of the GEMV form up to 64) and its
    # boundary (3 and 4 rows take the GEMV form up to K = 4096, the tile form above): one or two x
    # tiles, 1 to 24 windows of K (ring wrap and tails of every length), and N an odd multiple of 32
    # for about half the seeds (a last workgroup with one weight tile).
    rng = np.random.default_rng(1700 + seed)
    M = int(rng.choice([3, 4, 5, 6, 7, 11, 19, 31, 32, 33, 40, 57, 64]))
    K = 256 * int(rng.integers(1, 25))
    N = 32 * int(rng.integers(1, 41))
    return M, K, N


@pytest.mark.parametrize("seed", range(10))
def test_sweep_weight_tiles(seed):
    M, K, N = _tiles_shape(seed)
    c = synth.affine_case(M, K, N, seed=200 + seed)
    w, s, b, x = _affine_dev(c)
    y = B.qmm_affine4(w, s, b, x)
    torch.cuda.synchronize()
    acc, _ = oracle.affine(c["w"], c["scales"], c["biases"], c["x"], M, K, N)
    ms, mx = _affine_scales(c)
    _assert_within(_bf16_to_f64(y), acc, K, mx, ms, f"sweep weight tiles seed={seed} M={M} K={K} N={N}")


def _lut_shape(seed):
    rng = np.random.default_rng(2000 + seed)
    block = int(rng.choice([8, 16, 32, 64, 128]))
    M = int(rng.choice([2, 3, 7, 64, 130, 257]))
    K = max(32, block) * int(rng.integers(1, 9))
    K = K if K % 32 == 0 else K * 2
    N = int(rng.integers(8, 400))
    return M, K, N, block


@pytest.mark.parametrize("seed", SEEDS)
def test_sweep_lut_fp16(seed):
    M, K, N, block = _lut_shape(seed)
    c = synth.lut_case(M, K, N, seed=seed, block=block)
    x, p, s = _lut_dev(c)
    y = B.qmm_lut4(x, p, s, c["book"], N, block)
    torch.cuda.synchronize()
    acc, _ = oracle.lut4(c["x"], c["packed"], c["scales"], c["book"], M, K, N, block)
    got = y.float().cpu().numpy().astype(np.float64)
    _assert_within(got, acc, K, float(np.abs(oracle.f16_to_f32(c["x"])).max()),
                   float(np.abs(oracle.f16_to_f32(c["scales"])).max()),
                   f"sweep lut seed={seed} M={M} K={K} N={N} block={block}")


def _lut_vector_shape(seed):
    rng = np.random.default_rng(3000 + seed)
    block = int(rng.choice([2, 6, 8, 16, 24, 64]))
    M = int(rng.integers(1, 10))
    K = int(rng.integers(1, 700))
    N = int(rng.integers(1, 300))
    if seed % 2 == 0:  # every other case on the aligned forms' conditions
        K = block * max(1, K // block)
        N = block * max(1, N // block)
    return M, K, N, block


@pytest.mark.parametrize("seed", SEEDS)
def test_sweep_lut_weight_stored_k_by_n_fp16(seed):
    M, K, N, block = _lut_vector_shape(seed)
    rng = np.random.default_rng(seed)
    count = N * K
    packed = rng.integers(0, 256, (count + 1) // 2, dtype=np.uint16).astype(np.uint8)
    scales = oracle.f32_to_f16(rng.uniform(0.01, 0.05, -(-count // block)).astype(np.float32))
    x = oracle.f32_to_f16(rng.standard_normal((M, K)).astype(np.float32))
    book = synth.normal_codebook()
    y = B.qmm_lut4(_t(x.view(np.int16)).view(torch.float16), _t(packed), _t(scales.view(np.int16)).view(torch.float16),
                   book, N, block, transpose=0)
    acc, _ = oracle.lut4(x, packed, scales, book, M, K, N, block, transpose=False, round_half=True)
    got = y.float().cpu().numpy().astype(np.float64)
    _assert_within(got, acc, K, float(np.abs(oracle.f16_to_f32(x)).max()),
                   float(np.abs(oracle.f16_to_f32(scales)).max()),
                   f"sweep lut [K,N] seed={seed} M={M} K={K} N={N} block={block}")


@pytest.mark.parametrize("transpose", [0, 1])
@pytest.mark.parametrize("seed", SEEDS)
def test_sweep_lut_f32(seed, transpose):
    M, K, N, block = _lut_vector_shape(seed + 100 * transpose)
    x, packed, scales, book = _lut_f32_case(M, K, N, block, transpose, seed=seed)
    y = B.qmm_lut4_f32(_t(x), _t(packed), _t(scales), book, N, block, transpose=transpose).cpu().numpy()
    acc, _ = oracle.lut4_f32(x, packed, scales, book, M, K, N, block, bool(transpose))
    _assert_within(y.astype(np.float64), acc, K, float(np.abs(x).max()), float(np.abs(scales).max()),
                   f"sweep lut f32 seed={seed} M={M} K={K} N={N} block={block} t={transpose}")


@pytest.mark.parametrize("seed", SEEDS)
def test_sweep_moe(seed):
    rng = np.random.default_rng(4000 + seed)
    E = int(rng.integers(2, 21))
    N = int(rng.integers(16, 200))
    K = 64 * int(rng.integers(1, 17))            # 64 .. 1024
    T = int(rng.choice([1, 4, 17, 32, 33, 60, 120]))
    top_k = int(rng.integers(1, min(E, 8) + 1))
    c = synth.moe_case(E, N, K, T, top_k, seed=seed)
    got, scratch = _moe_run(c)
    acc, _ = oracle.moe_q4_0(c["x"], c["w"], c["ids"], T, top_k, N, K, E, c["expert_stride"])
    _assert_within(got, acc, K, float(np.abs(c["x"]).max()), _max_d(c),
                   f"sweep moe seed={seed} E={E} N={N} K={K} T={T} top_k={top_k}")
    assert scratch[:4].view(torch.int32).item() == 0
