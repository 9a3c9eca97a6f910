"""Parity at the documented size limits, every output against the oracle.

The affine entry points are implemented for K and N up to 2^21: the decode GEMV, the weight-tile
form (also for two rows, which past K = 8192 take it), the prefill tiles and the 64x128 kernel
are run with K = 2^21 or N = 2^21. The lookup entry points take M up to 262,140 (4 rows per
workgroup times the 65,535 workgroups of a grid's y dimension on the `[K, N]` vector kernels);
that M is run on those kernels and on both matrix-core routes. The expert-routed entry point
groups up to 8192 experts; every route runs at that count. Shapes past these limits are rejected
before any launch (tests/test_abi_host.py).
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

KMAX = NMAX = 1 << 21
MMAX_LUT = 4 * 65535

AFFINE = [
    (1, KMAX, 64),          # decode GEMV, K at the limit
    (1, 64, NMAX),          # decode GEMV, N at the limit
    (2, KMAX, 64),          # two rows past K = 8192: the weight-tile form
    (8, KMAX, 64),          # weight tiles, 8192 windows
    (8, 256, NMAX),         # weight tiles, 32768 workgroups
    (65, KMAX, 32),         # prefill tiles, K at the limit
    (65, 64, NMAX),         # prefill tiles, N at the limit
    (40, KMAX - 64, 32),    # K % 256 != 0: the 64x128 kernel
]


@pytest.mark.parametrize("M,K,N", AFFINE)
def test_affine_at_the_size_limits(M, K, N):
    print(f"limits affine M={M} K={K} N={N}", flush=True)
    c = synth.affine_case(M, K, N, seed=41)
    w, s, b, x = _affine_dev(c)
    y = (B.qmv_affine4 if M == 1 else B.qmm_affine4)(w, s, b, x)
    torch.cuda.synchronize()
    acc, _ = oracle.affine(c["w"], c["scales"], c["biases"], c["x"], M, K, N)
    ms, mx = _affine_scales(c)
    _assert_within(_bf16_to_f64(y), acc, K, mx, ms, f"limits affine M={M} K={K} N={N}")


# (K, N, block, transpose): the [K, N] vector kernels (K % 64 != 0) on a grid of 65,535
# workgroups in y, the [K, N] matrix-core route, the [N, K] matrix-core route
LUT = [(40, 24, 8, 0), (64, 8, 8, 0), (32, 8, 8, 1)]


@pytest.mark.parametrize("K,N,block,transpose", LUT)
def test_lut4_at_the_row_limit(K, N, block, transpose):
    M = MMAX_LUT
    print(f"limits lut4 M={M} K={K} N={N} block={block} transpose={transpose}", flush=True)
    c = synth.lut_case(M, K, N, seed=42, block=block)
    x, p, s = _lut_dev(c)
    y = B.qmm_lut4(x, p, s, c["book"], N, block, transpose=transpose)
    torch.cuda.synchronize()
    acc, _ = oracle.lut4(c["x"], c["packed"], c["scales"], c["book"], M, K, N, block, transpose=bool(transpose))
    _assert_within(y.float().cpu().numpy().astype(np.float64), acc, K, float(np.abs(oracle.f16_to_f32(c["x"])).max()),
                   float(np.abs(oracle.f16_to_f32(c["scales"])).max()),
                   f"limits lut4 M={M} K={K} N={N} block={block} transpose={transpose}")


@pytest.mark.parametrize("transpose", [0, 1])
def test_lut4_f32_at_the_row_limit(transpose):
    M, K, N, block = MMAX_LUT, 24, 16, 8
    print(f"limits lut4_f32 M={M} transpose={transpose}", flush=True)
    x, packed, scales, book = _lut_f32_case(M, K, N, block, transpose, seed=43)
    y = B.qmm_lut4_f32(_t(x), _t(packed), _t(scales), book, N, block, transpose=transpose).cpu().numpy()
    acc, _ = oracle.lut4_f32(x, packed, scales, book, M, K, N, block, bool(transpose))
    _assert_within(y.astype(np.float64), acc, K, float(np.abs(x).max()), float(np.abs(scales).max()),
                   f"limits lut4_f32 M={M} transpose={transpose}")


# (tokens, top_k) at the most experts the grouped routes take (8192): the mat-vec route, the
# one-launch grouped GEMM (512 routed rows) and the two-launch form (4800 routed rows, the
# grouping kernel's per-expert counters at their largest)
@pytest.mark.parametrize("T,top_k", [(4, 8), (64, 8), (600, 8)])
def test_moe_at_the_expert_limit(T, top_k):
    E, N, K = 8192, 32, 64
    print(f"limits moe E={E} N={N} K={K} T={T} top_k={top_k}", flush=True)
    c = synth.moe_case(E, N, K, T, top_k, seed=44)
    c["ids"][: top_k] = np.arange(E - top_k, E, dtype=np.uint32)  # the highest expert ids are used
    got, scratch = _moe_run(c)
    acc, _ = oracle.moe_q4_0(c["x"], c["w"], c["ids"], T, top_k, N, K, E, c["expert_stride"])
    _assert_within(got, acc, K, float(np.abs(c["x"]).max()), _max_d(c),
                   f"limits moe E={E} T={T} top_k={top_k}")
    assert scratch[:4].view(torch.int32).item() == 0
