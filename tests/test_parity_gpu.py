"""GPU parity: the HIP library against the CPU oracle on identical seeded inputs.

Bar: unpacked nibbles / codebook indices / Q4_0 codes and scales bit-exact;
outputs within |y - ref| <= 1e-2 |ref| + 1e-2 sqrt(K) max|x| max|scale|, with
ref the oracle's fp64 accumulator. Small shapes are compared element by
element (spanning several tiles and ragged tails); the full-size workloads in
the launch configuration the benchmark times are compared at sampled outputs
the oracle computes one by one.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from weight_only_bit_w4_amd import binding as B
from weight_only_bit_w4_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _t(a: np.ndarray, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def _affine_dev(c):
    return (_t(c["w"].view(np.int32)), _t(c["scales"].view(np.int16), torch.bfloat16),
            _t(c["biases"].view(np.int16), torch.bfloat16), _t(c["x"].view(np.int16), torch.bfloat16))


def _bf16_to_f64(y: torch.Tensor) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)


def _assert_within(got, ref, K, max_x, max_s, what):
    tol = oracle.tolerance(ref, K, max_x, max_s)
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst err {err.max():.3g} "
                           f"(tol there {tol.reshape(-1)[np.argmax(err)]:.3g})")


def _affine_scales(c):
    return float(np.abs(oracle.bf16_to_f32(c["scales"])).max()), float(np.abs(oracle.bf16_to_f32(c["x"])).max())


# ---------------------------------------------------------------- unpack, bit-exact
@pytest.mark.parametrize("N,K", [(256, 256), (96, 40), (4096, 4096), (14336, 4096)])
def test_unpack_affine_bit_exact(N, K):
    c = synth.affine_case(1, K, N, seed=11)
    q = B.w4_unpack_affine(_t(c["w"].view(np.int32)), N, K).cpu().numpy()
    assert np.array_equal(q, oracle.unpack_affine(c["w"], N, K))


@pytest.mark.parametrize("N,K", [(48, 128), (11008, 4096)])
def test_unpack_lut_bit_exact(N, K):
    c = synth.lut_case(1, K, N, seed=12)
    codes = B.w4_unpack_lut(_t(c["packed"]), N * K).cpu().numpy()
    assert np.array_equal(codes, oracle.unpack_lut(c["packed"], N * K))


@pytest.mark.parametrize("E,N,K", [(3, 20, 128), (64, 1408, 2048)])
def test_unpack_q4_0_bit_exact(E, N, K):
    c = synth.moe_case(E, N, K, 1, 1, seed=13)
    q, d = B.w4_unpack_q4_0(_t(c["w"]), E * N, K)
    q_ref, d_ref = oracle.unpack_q4_0(c["w"], E * N, K)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(oracle.f16_to_f32(d.cpu().numpy().view(np.uint16)), d_ref)


# ---------------------------------------------------------------- decode GEMV
@pytest.mark.parametrize("K,N,seed", [
    (256, 256, 0),        # the tiny workload's weights, one row of x
    (96, 64, 1),          # fewer groups than lanes
    (4096 + 32, 96, 2),   # a ragged second chunk of groups
    (10240, 64, 3),       # more chunks than the unrolled forms (runtime loop)
    (8192, 64, 4),        # the largest shared-x form: 4 chunks
    (8224, 32, 5),        # one group past it: the runtime loop with a 1-group last chunk
    (2080, 160, 6),       # 2 chunks, the second holding one group; 10 workgroups of 16 rows
    (4096, 14336, 0),     # the decode workload at full size
])
def test_qmv_affine4(K, N, seed):
    c = synth.affine_case(1, K, N, seed=seed)
    w, s, b, x = _affine_dev(c)
    y = B.qmv_affine4(w, s, b, x)
    torch.cuda.synchronize()
    acc, _ = oracle.affine(c["w"], c["scales"], c["biases"], c["x"], 1, K, N)
    ms, mx = _affine_scales(c)
    _assert_within(_bf16_to_f64(y), acc, K, mx, ms, f"qmv K={K} N={N}")


# ---------------------------------------------------------------- prefill GEMM
@pytest.mark.parametrize("M,K,N", [
    (4, 256, 256),                        # the tiny workload
    (32, 32, 32), (4, 32, 32), (7, 64, 64), (64, 32, 32), (64, 128, 256), (100, 256, 512),  # page's test shapes
    (300, 160, 224),                      # ragged M, N not a multiple of the 128 tile
    (65, 96, 160),                        # just past the small-M tile
    (260, 192, 96),                       # K % 64 == 0 prefill path: 3 K steps (ring wrap), ragged M and N
    (513, 320, 416),                      # 5 K steps, M one past two 256-row tiles
    (256, 64, 128),                       # a single K step, exact tiles
    (300, 128, 256),                      # 2 K steps (producer loop tail of 2)
    (257, 256, 160),                      # 4 K steps (one unrolled round + a tail of 1)
    (384, 1024, 384),                     # 16 K steps, several tiles each way
    # K % 256 == 0: scales and biases come four steps to a load, the producer loop unrolled by 12
    (300, 768, 160),                      # 12 K steps: one unrolled round, no tail
    (270, 2048, 96),                      # 32 K steps: two rounds and a tail of 8
    (520, 5120, 224),                     # 80 K steps: six rounds and a tail of 8, three row tiles
    # the GEMV form (every weight row read once for all rows): the rows it applies in one pass (4
    # for K <= 4096, 2 above), or up to 16 rows when K % 256 != 0 (K <= 8192)
    (2, 4096, 14336),                     # the decode workload's weights, two rows (batches of 2)
    (4, 4096, 256),                       # one pass of 4 rows: the GEMV form
    (2, 8192, 64),                        # K > 4096, one pass of 2 rows: the GEMV form
    (5, 4096, 256),                       # two passes: the weight-tile form instead
    (3, 8192, 64),                        # K > 4096, two passes of 2: the weight-tile form
    (3, 96, 64),                          # 3 groups, one batch of 4 with a missing row
    (5, 2080, 160),                       # ragged second chunk, a 1-row second batch
    (8, 4160, 256),                       # 3 chunks: batches of 2
    (12, 2112, 96),                       # 2 chunks, batches of 4
    (16, 4128, 160),                      # 3 chunks, batches of 2
    (13, 8160, 32),                       # 4 chunks, batches of 2, a 1-row last batch
    (6, 8224, 32),                        # one group past the GEMV form: the matrix-core path
    (40, 96, 96),                         # 3 K steps: the load ring's prologue covers all of K
    (64, 544, 256),                       # 17 K steps: ring wrap with a partial last round
    # 6 <= M <= 64 with K % 256 == 0: weight tiles streamed once (256-wide K windows; a
    # 6-slot ring for up to 32 rows of x, 3 slots above)
    (6, 256, 64),                         # the smallest M of the tile form, one window
    (8, 4096, 256),                       # 16 windows: two rounds of 6 and a tail of 4
    (8, 8192, 64),                        # 32 windows, one workgroup
    (6, 6144, 96),                        # 24 windows (four full rounds), a half workgroup
    (16, 4096, 160),                      # ragged last workgroup (32 rows)
    (13, 8192, 32),                       # one tile: the second tile's rows are past N
    (17, 4096, 14336),                    # the decode workload's weights, 17 rows
    (20, 1536, 224),                      # 6 windows (exactly one round), 3.5 workgroups
    (31, 3328, 32),                       # 13 windows, one tile
    (33, 768, 160),                       # two x tiles (3-slot ring): 3 windows, 2.5 workgroups
    (48, 512, 4096),                      # two x tiles, 2 windows, 64 workgroups
    (64, 2816, 96),                       # two x tiles, 11 windows: three rounds and a tail of 2
])
def test_qmm_affine4_small(M, K, N):
    c = synth.affine_case(M, K, N, seed=M + K + N)
    w, s, b, x = _affine_dev(c)
    y = B.qmm_affine4(w, s, b, x)
    torch.cuda.synchronize()
    acc, _ = oracle.affine(c["w"], c["scales"], c["biases"], c["x"], M, K, N)
    ms, mx = _affine_scales(c)
    _assert_within(_bf16_to_f64(y), acc, K, mx, ms, f"qmm M={M} K={K} N={N}")


# Short K on every route of qmm_affine4, element by element: the GEMV forms (the rows one pass takes,
# 4 up to K = 4096, and M <= 16 with K % 256 != 0), the 64x128-tile kernel (17 <= M <= 64 with
# K % 256 != 0), the register-staged prefill kernel (M > 64, K % 64 == 32), the specialised-wavefront
# prefill kernel (M > 64, K % 64 == 0) and the weight-tile kernel (past one GEMV pass up to 64 rows,
# K % 256 == 0). Small K is where operand rounding weighs most against the bound (few products, small
# |ref|).
@pytest.mark.parametrize("M,K,N", [(m, k, n) for k, n in ((32, 96), (64, 128), (96, 160))
                                   for m in (2, 5, 6, 12, 16, 17, 40, 64, 65, 100, 300)]
                         + [(4, 256, 64), (5, 256, 64), (6, 256, 96), (20, 256, 128), (40, 512, 64),
                            (64, 256, 160)])
def test_qmm_affine4_short_k_every_route(M, K, N):
    c = synth.affine_case(M, K, N, seed=7 * M + K + N)
    w, s, b, x = _affine_dev(c)
    y = B.qmm_affine4(w, s, b, x)
    torch.cuda.synchronize()
    acc, _ = oracle.affine(c["w"], c["scales"], c["biases"], c["x"], M, K, N)
    ms, mx = _affine_scales(c)
    _assert_within(_bf16_to_f64(y), acc, K, mx, ms, f"qmm short K M={M} K={K} N={N}")


# Operand range of the binary16 routes: a finite x (or weight) that binary16 cannot hold makes its output
# row (or column) non-finite and is counted; an infinite x propagates and is not counted. The GEMV forms
# (bf16 products, f32 scale and bias) hold such values exactly.
_BF16_1E5 = 0x47C3      # 99840.0, finite in bf16, beyond binary16's 65504
_BF16_INF = 0x7F80


@pytest.mark.parametrize("M,K,N,route", [
    (300, 256, 256, "specialised-wavefront prefill"),
    (300, 96, 128, "register-staged prefill"),
    (40, 96, 128, "64x128 tile"),
    (20, 512, 128, "weight tile"),
])
def test_qmm_affine4_range_events(M, K, N, route):
    c = synth.affine_case(M, K, N, seed=31)
    x = c["x"].copy()
    x[3, 17] = _BF16_1E5
    x[5, 0] = _BF16_INF
    scales = c["scales"].copy()
    scales[7, 1] = 0x4600     # 8192: q * s + b reaches ~122880 for q = 15
    biases = c["biases"].copy()
    biases[7, 1] = 0
    w, s, b, xd = _affine_dev(dict(c, x=x, scales=scales, biases=biases))
    B.w4_range_events(reset=True)
    y = B.qmm_affine4(w, s, b, xd)
    events = B.w4_range_events(reset=True)
    yf = _bf16_to_f64(y)
    assert events >= 1, route
    assert not np.isfinite(yf[3]).any() and not np.isfinite(yf[5]).any(), route
    assert not np.isfinite(yf[:, 7]).any(), route
    keep_m = np.setdiff1d(np.arange(M), [3, 5])
    keep_n = np.setdiff1d(np.arange(N), [7])
    acc, _ = oracle.affine(c["w"], scales, biases, x, M, K, N)
    ms = float(np.abs(oracle.bf16_to_f32(c["scales"])).max())
    mx = float(np.abs(oracle.bf16_to_f32(c["x"])).max())
    _assert_within(yf[np.ix_(keep_m, keep_n)], acc[np.ix_(keep_m, keep_n)], K, mx, ms, f"range {route}")


def test_qmm_affine4_range_clean_inputs_and_infinities_are_not_counted():
    M, K, N = 300, 256, 256
    c = synth.affine_case(M, K, N, seed=32)
    x = c["x"].copy()
    x[9, 40] = _BF16_INF
    w, s, b, xd = _affine_dev(dict(c, x=x))
    B.w4_range_events(reset=True)
    y = B.qmm_affine4(w, s, b, xd)
    assert B.w4_range_events(reset=True) == 0
    yf = _bf16_to_f64(y)
    assert not np.isfinite(yf[9]).any()
    assert np.isfinite(np.delete(yf, 9, axis=0)).all()


def test_qmm_affine4_gemv_forms_hold_large_x_exactly():
    M, K, N = 3, 256, 96
    c = synth.affine_case(M, K, N, seed=33)
    x = c["x"].copy()
    x[1, 5] = _BF16_1E5
    w, s, b, xd = _affine_dev(dict(c, x=x))
    B.w4_range_events(reset=True)
    y = B.qmm_affine4(w, s, b, xd)
    assert B.w4_range_events(reset=True) == 0
    acc, _ = oracle.affine(c["w"], c["scales"], c["biases"], x, M, K, N)
    ms, mx = _affine_scales(c)   # max |x| without the planted value: the bound stays as tight as for plain x
    _assert_within(_bf16_to_f64(y), acc, K, mx, ms, "GEMV form with a large x")


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N", [(24, 512, 96), (5, 4096, 64)])
def test_qmm_affine4_small_unaligned_scales(M, K, N):
    """Scales and biases only 2-byte aligned: the weight-tile form (4-byte DMA offsets) is not
    taken; the 64x128-tile matrix-core kernel (24 rows) or the GEMV form in two passes (5 rows)
    gives the same result."""
    c = synth.affine_case(M, K, N, seed=5)
    w, s, b, x = _affine_dev(c)
    s2 = torch.empty(s.numel() + 1, dtype=torch.bfloat16, device="cuda")[1:].view(N, K // 32)
    b2 = torch.empty(b.numel() + 1, dtype=torch.bfloat16, device="cuda")[1:].view(N, K // 32)
    s2.copy_(s)
    b2.copy_(b)
    assert s2.data_ptr() % 4 == 2 and b2.data_ptr() % 4 == 2
    y = B.qmm_affine4(w, s2, b2, x)
    torch.cuda.synchronize()
    acc, _ = oracle.affine(c["w"], c["scales"], c["biases"], c["x"], M, K, N)
    ms, mx = _affine_scales(c)
    _assert_within(_bf16_to_f64(y), acc, K, mx, ms, "qmm unaligned scales")


def _sample_points(M, N, count, seed, tile_m=256, tile_n=128):
    rng = np.random.default_rng(seed)
    ms = rng.integers(0, M, count)
    ns = rng.integers(0, N, count)
    corners_m = np.array([0, M - 1, tile_m - 1, tile_m, min(M - 1, 2 * tile_m + 17)])
    corners_n = np.array([0, N - 1, tile_n - 1, tile_n, min(N - 1, 3 * tile_n + 5)])
    cm, cn = np.meshgrid(corners_m, corners_n)
    return np.concatenate([ms, cm.reshape(-1)]), np.concatenate([ns, cn.reshape(-1)])


def test_qmm_affine4_prefill_full_size_sampled():
    c = synth.prefill_affine()
    M, K, N = c["M"], c["K"], c["N"]
    w, s, b, x = _affine_dev(c)
    y = B.qmm_affine4(w, s, b, x)
    torch.cuda.synchronize()
    ms, ns = _sample_points(M, N, 3000, seed=21)
    acc, _ = oracle.affine_points(c["w"], c["scales"], c["biases"], c["x"], K, ms, ns)
    got = _bf16_to_f64(y)[ms, ns]
    msc, mx = _affine_scales(c)
    _assert_within(got, acc, K, mx, msc, "qmm prefill sampled")
    assert torch.isfinite(y.float()).all()


def test_qmm_affine4_prefill_full_size_every_output():
    """The prefill workload (M=2048, K=N=4096) in the launch configuration the benchmark times, every one
    of its 8.39 M outputs against the oracle (the XCD-aware tile order is only taken at this size)."""
    c = synth.prefill_affine()
    M, K, N = c["M"], c["K"], c["N"]
    w, s, b, x = _affine_dev(c)
    B.w4_range_events(reset=True)
    y = B.qmm_affine4(w, s, b, x)
    torch.cuda.synchronize()
    acc, _ = oracle.affine(c["w"], c["scales"], c["biases"], c["x"], M, K, N)
    msc, mx = _affine_scales(c)
    _assert_within(_bf16_to_f64(y), acc, K, mx, msc, "qmm prefill every output")
    assert B.w4_range_events(reset=True) == 0


# The prefill tiles in XCD blocks: each of the 8 XCDs takes a block of (tiles_m / pm) x (tiles_n / pn)
# tiles, pm * pn = 8, the split that reads the fewest bytes. Each split (pm = 1, 2, 4, 8) on each
# prefill kernel (K % 256 == 0, K % 64 == 0, and the register-staged one for K % 64 == 32), with
# blocks of one tile and of several, and ragged last row and column tiles.
@pytest.mark.parametrize("M,K,N", [
    (256, 64, 1024), (512, 64, 512), (1024, 64, 256), (2048, 64, 128),   # pm = 1, 2, 4, 8: one tile per XCD
    (200, 256, 2016),                     # pm = 1, 2 tiles per XCD, K % 256 == 0
    (500, 64, 2016), (300, 128, 4064),    # pm = 2, ragged M and N
    (1000, 320, 992), (1000, 256, 1984),  # pm = 4, 4 and 8 tiles per XCD
    (1800, 192, 480), (4000, 64, 96),     # pm = 8, 2 tiles per XCD
    (130, 160, 1024), (260, 96, 992), (1020, 480, 992), (2000, 96, 224),  # register-staged: pm = 1, 2, 4, 8
])
def test_qmm_affine4_prefill_xcd_blocks(M, K, N):
    c = synth.affine_case(M, K, N, seed=M + N + K)
    w, s, b, x = _affine_dev(c)
    y = B.qmm_affine4(w, s, b, x)
    torch.cuda.synchronize()
    acc, _ = oracle.affine(c["w"], c["scales"], c["biases"], c["x"], M, K, N)
    ms, mx = _affine_scales(c)
    _assert_within(_bf16_to_f64(y), acc, K, mx, ms, f"prefill xcd blocks M={M} K={K} N={N}")


def test_affine_m_zero_is_noop():
    c = synth.affine_case(2, 64, 32, seed=5)
    w, s, b, _ = _affine_dev(c)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    y = B.qmm_affine4(w, s, b, x)
    assert y.shape == (0, 32)


@pytest.mark.parametrize("transpose", [1, 0])
@pytest.mark.parametrize("f32", [False, True])
def test_lut_m_zero_is_noop(f32, transpose):
    M, K, N, block = 0, 64, 48, 16
    c = synth.lut_case(2, K, N, seed=6, block=block)
    if f32:
        x = torch.empty((M, K), dtype=torch.float32, device=DEV)
        p, s = _t(c["packed"]), _t(oracle.f16_to_f32(c["scales"]))
        y = B.qmm_lut4_f32(x, p, s, c["book"], N, block, transpose=transpose)
    else:
        x = torch.empty((M, K), dtype=torch.float16, device=DEV)
        _, p, s = _lut_dev(c)
        y = B.qmm_lut4(x, p, s, c["book"], N, block, transpose=transpose)
    torch.cuda.synchronize()
    assert y.shape == (0, N)


# ---------------------------------------------------------------- lookup codebook
def _lut_dev(c):
    return _t(c["x"].view(np.int16), torch.float16), _t(c["packed"]), _t(c["scales"].view(np.int16), torch.float16)


@pytest.mark.parametrize("M,K,N,block", [
    (5, 128, 48, 64), (70, 256, 200, 64), (300, 64, 130, 32), (3, 64, 16, 8),
    (260, 320, 300, 16),     # 5 K steps, two scales per K step, ragged M and N
    (513, 384, 96, 128),     # 6 K steps, one scale per two steps, M one past two 256-row tiles
    (72, 192, 1000, 8),      # block 8: the general path
])
def test_qmm_lut4_small(M, K, N, block):
    c = synth.lut_case(M, K, N, seed=M + N, block=block)
    x, p, s = _lut_dev(c)
    y = B.qmm_lut4(x, p, s, c["book"], N, block)
    torch.cuda.synchronize()
    acc, _ = oracle.lut4(c["x"], c["packed"], c["scales"], c["book"], M, K, N, block)
    got = y.float().cpu().numpy().astype(np.float64)
    _assert_within(got, acc, K, float(np.abs(oracle.f16_to_f32(c["x"])).max()),
                   float(np.abs(oracle.f16_to_f32(c["scales"])).max()), f"lut M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N,block", [
    (4, 256, 96, 64),      # aligned column form: N a multiple of the block
    (3, 100, 70, 6),       # blocks straddle rows: element-by-element form
    (130, 64, 250, 16),    # more than 128 rows of x but N % 8 != 0: the vector route, 33 row groups of 4
    (2, 5000, 40, 10),     # K split over 16 wavefronts with a ragged last range
    (5, 1000, 200, 8),     # dword form: a partial last 64-column group, ragged K
    (4, 4096, 11008, 64),  # dword form on the LUT workload's weights
    # matrix-core route (M >= 128, K % 64 == 0, N % 8 == 0, power-of-two block >= 8)
    (130, 64, 256, 16),    # one K step, ragged M
    (128, 64, 96, 8),      # one tile, the smallest block
    (300, 192, 200, 32),   # 3 K steps, ragged M and N (200 of 288 tile columns)
    (257, 320, 104, 256),  # blocks longer than a row straddle rows; M one past a tile
    (200, 192, 1000, 1024),  # a partial last block (N K / block = 187.5)
])
def test_qmm_lut4_weight_stored_k_by_n(M, K, N, block):
    _lut_kn_check(M, K, N, block)


def test_qmm_lut4_weight_stored_k_by_n_full_size_every_output():
    """The lookup workload's shape (M=512, K=4096, N=11008, block 64) with W stored [K, N]: the
    matrix-core route, every output against the oracle."""
    _lut_kn_check(512, 4096, 11008, 64)


def _lut_kn_check(M, K, N, block):
    # Half-precision path with transpose == 0 (W stored [K, N], flat = k * N + n).
    rng = np.random.default_rng(M + K)
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
                   float(np.abs(oracle.f16_to_f32(scales)).max()), f"lut [K,N] M={M} K={K} N={N} block={block}")


def test_qmm_lut4_full_size_sampled():
    c = synth.lut_matmul_case()
    M, K, N, block = c["M"], c["K"], c["N"], c["block"]
    x, p, s = _lut_dev(c)
    y = B.qmm_lut4(x, p, s, c["book"], N, block)
    torch.cuda.synchronize()
    ms, ns = _sample_points(M, N, 3000, seed=22)
    acc = oracle.lut4_points(c["x"], c["packed"], c["scales"], c["book"], K, block, ms, ns)
    got = y.float().cpu().numpy().astype(np.float64)[ms, ns]
    _assert_within(got, acc, K, float(np.abs(oracle.f16_to_f32(c["x"])).max()),
                   float(np.abs(oracle.f16_to_f32(c["scales"])).max()), "lut full sampled")


def test_qmm_lut4_full_size_every_output():
    """The lookup workload (M=512, K=4096, N=11008, block 64), every output against the oracle."""
    c = synth.lut_matmul_case()
    M, K, N, block = c["M"], c["K"], c["N"], c["block"]
    x, p, s = _lut_dev(c)
    y = B.qmm_lut4(x, p, s, c["book"], N, block)
    torch.cuda.synchronize()
    acc, _ = oracle.lut4(c["x"], c["packed"], c["scales"], c["book"], M, K, N, block)
    got = y.float().cpu().numpy().astype(np.float64)
    _assert_within(got, acc, K, float(np.abs(oracle.f16_to_f32(c["x"])).max()),
                   float(np.abs(oracle.f16_to_f32(c["scales"])).max()), "lut every output")


# ---------------------------------------------------------------- expert-routed Q4_0
def _moe_run(c, ids=None):
    ids = c["ids"] if ids is None else ids
    x, w, idt = _t(c["x"]), _t(c["w"]), _t(ids.view(np.int32))
    scratch = torch.empty(B.qmm_id_q4_0_scratch_bytes(c["n_experts"], c["n_tokens"], c["top_k"], c["K"]),
                          dtype=torch.uint8, device=DEV)
    out = B.qmm_id_q4_0(x, w, idt, c["n_tokens"], c["top_k"], c["N"], c["K"], c["n_experts"], c["expert_stride"],
                        scratch=scratch)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), scratch


def _max_d(c):
    E, N, K = c["n_experts"], c["N"], c["K"]
    _, d = oracle.unpack_q4_0(c["w"], E * N, K)
    return float(np.abs(d).max())


@pytest.mark.parametrize("E,N,K,T,top_k", [
    # grouped GEMM route (more than 32 tokens)
    (4, 40, 128, 33, 2),     # one token past the mat-vec threshold; N not a multiple of the 128-row tile
    (2, 64, 64, 100, 2),     # 100 routed rows per expert: two passes of 64
    (8, 200, 320, 40, 3),    # K not a multiple of the 256 window
    (16, 96, 256, 32, 9),    # 32 tokens but 288 routed rows: past the mat-vec id scan
    (2500, 16, 64, 40, 2),   # more experts than grouping threads: 3 experts per scan segment
    (16, 64, 128, 288, 8),   # 2304 routed rows, 144 per expert: five passes of 32
    (5, 64, 128, 461, 5),    # 2305 routed rows over 5 experts: a last pass of 1 row for some
    (16, 64, 128, 600, 8),   # 4800 routed rows: past the one-launch route, grouped in scratch first
    (8, 96, 96, 700, 6),     # 4200 routed rows with 3 blocks per row: the two-launch realigning form
    # mat-vec route (at most 32 tokens)
    (4, 40, 128, 3, 2),      # tiny, N not a multiple of the 32-row tile
    (8, 200, 320, 9, 3),     # 10 blocks: a ragged first chunk
    (6, 33, 96, 4, 1),       # K % 64 != 0 (3 blocks), top_k 1, 33 rows: a 1-row last tile
    (5, 64, 8192, 2, 3),     # 4 chunks of 64 blocks, the most the route takes
    (64, 1408, 2048, 1, 8),  # one decode token of the MoE workload's shapes
    (64, 1408, 2048, 32, 8), # at the threshold: 256 routed rows, experts shared between tokens
])
def test_qmm_id_q4_0_small(E, N, K, T, top_k):
    c = synth.moe_case(E, N, K, T, top_k, seed=E + N + T)
    got, scratch = _moe_run(c)
    acc, _ = oracle.moe_q4_0(c["x"], c["w"], c["ids"], T, top_k, N, K, E, c["expert_stride"])
    _assert_within(got, acc, K, float(np.abs(c["x"]).max()), _max_d(c), f"moe E={E} N={N} K={K} T={T}")
    assert scratch[:4].view(torch.int32).item() == 0


@pytest.mark.parametrize("T", [5, 40, 800])  # mat-vec route, grouped GEMM (few and many rows per expert)
def test_qmm_id_q4_0_duplicate_and_out_of_range_ids(T):
    c = synth.moe_case(4, 32, 64, T, 3, seed=31)
    ids = c["ids"].copy()
    ids[1] = ids[0]          # the same expert twice for token 0
    ids[4] = 9               # no such expert
    ids[10] = 0xFFFFFFFF
    ids[13] = 9              # the same missing expert again
    got, scratch = _moe_run(c, ids)
    acc, _ = oracle.moe_q4_0(c["x"], c["w"], ids, T, 3, 32, 64, 4, c["expert_stride"])
    _assert_within(got, acc, 64, float(np.abs(c["x"]).max()), _max_d(c), f"moe odd ids T={T}")
    assert np.all(got[4] == 0) and np.all(got[10] == 0) and np.all(got[13] == 0)
    assert scratch[:4].view(torch.int32).item() == 3


@pytest.mark.parametrize("K", [8256, 8224])
def test_qmm_id_q4_0_mat_vec_route_limits(K):
    # Past 4 chunks (K > 8192) a few tokens go to the grouped GEMM, with an even and an odd block count.
    c = synth.moe_case(2, 32, K, 2, 2, seed=K)
    got, _ = _moe_run(c)
    acc, _ = oracle.moe_q4_0(c["x"], c["w"], c["ids"], 2, 2, 32, K, 2, c["expert_stride"])
    _assert_within(got, acc, K, float(np.abs(c["x"]).max()), _max_d(c), f"moe K={K}")


@pytest.mark.parametrize("E,N,K,T,top_k", [
    (8, 96, 96, 40, 2),      # 3 blocks: one window, 3 live blocks
    (4, 72, 160, 50, 3),     # 5 blocks: a last window of 1
    (6, 200, 224, 64, 2),    # 7 blocks, N not a multiple of the tile
    (3, 400, 2080, 40, 2),   # 65 blocks (17 windows), two row chunks (384 + 16)
])
def test_qmm_id_q4_0_grouped_odd_block_rows(E, N, K, T, top_k):
    """Grouped route with K % 64 == 32: every other weight row starts 2 bytes past a dword."""
    c = synth.moe_case(E, N, K, T, top_k, seed=E * K + T)
    got, scratch = _moe_run(c)
    acc, _ = oracle.moe_q4_0(c["x"], c["w"], c["ids"], T, top_k, N, K, E, c["expert_stride"])
    _assert_within(got, acc, K, float(np.abs(c["x"]).max()), _max_d(c), f"moe odd blocks E={E} N={N} K={K}")
    assert scratch[:4].view(torch.int32).item() == 0


def _restride(c, pad):
    """c's weights with `pad` bytes between expert slabs (none after the last)."""
    E, slab = c["n_experts"], c["expert_stride"]
    w = np.zeros((E - 1) * (slab + pad) + slab, np.uint8)
    for e in range(E):
        w[e * (slab + pad):e * (slab + pad) + slab] = c["w"][e * slab:(e + 1) * slab]
    return dict(c, w=w, expert_stride=slab + pad)


@pytest.mark.parametrize("T", [5, 40])   # the mat-vec route and the grouped route
@pytest.mark.parametrize("K,pad,offset", [
    (128, 2, 0),    # expert stride 2 mod 4
    (128, 0, 2),    # w itself only 2-byte aligned
    (96, 2, 2),     # both, with an odd block count
    (256, 6, 2),    # both, 4-byte multiples of rows
])
def test_qmm_id_q4_0_two_byte_aligned_weights(T, K, pad, offset):
    E, N, top_k = 5, 72, 2
    base = synth.moe_case(E, N, K, T, top_k, seed=K + pad + offset + T)
    c = _restride(base, pad)
    buf = torch.zeros(c["w"].size + 16, dtype=torch.uint8, device=DEV)
    w = buf[offset:offset + c["w"].size]
    w.copy_(torch.from_numpy(c["w"]).to(DEV))
    assert w.data_ptr() % 4 == offset % 4
    x, idt = _t(c["x"]), _t(c["ids"].view(np.int32))
    out = B.qmm_id_q4_0(x, w, idt, T, top_k, N, K, E, c["expert_stride"])
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    acc, _ = oracle.moe_q4_0(c["x"], c["w"], c["ids"], T, top_k, N, K, E, c["expert_stride"])
    _assert_within(got, acc, K, float(np.abs(c["x"]).max()), _max_d(base), f"moe K={K} pad={pad} offset={offset} T={T}")


def test_qmm_id_q4_0_full_size_sampled():
    c = synth.moe_q4_0_case()
    got, scratch = _moe_run(c)
    rng = np.random.default_rng(23)
    rows = c["n_tokens"] * c["top_k"]
    rs = np.concatenate([rng.integers(0, rows, 3000), [0, rows - 1]])
    ns = np.concatenate([rng.integers(0, c["N"], 3000), [c["N"] - 1, 0]])
    acc = oracle.moe_q4_0_points(c["x"], c["w"], c["ids"], c["top_k"], c["K"], c["n_experts"], c["expert_stride"],
                                 rs, ns)
    _assert_within(got[rs, ns], acc, c["K"], float(np.abs(c["x"]).max()), _max_d(c), "moe full sampled")
    assert np.isfinite(got).all()


def test_qmm_id_q4_0_full_size_every_output():
    """The MoE workload (64 experts, N=1408, K=2048, 128 tokens, top-8), every routed row's outputs
    against the oracle, and no out-of-range id counted."""
    c = synth.moe_q4_0_case()
    got, scratch = _moe_run(c)
    acc, _ = oracle.moe_q4_0(c["x"], c["w"], c["ids"], c["n_tokens"], c["top_k"], c["N"], c["K"], c["n_experts"],
                             c["expert_stride"])
    _assert_within(got, acc, c["K"], float(np.abs(c["x"]).max()), _max_d(c), "moe every output")
    assert int(scratch[:4].cpu().numpy().view(np.uint32)[0]) == 0


@pytest.mark.parametrize("T", [3, 40])   # the mat-vec route and the grouped route
def test_qmm_id_q4_0_range_events(T):
    """A finite x beyond binary16's range is counted as a range event and its token's routed rows come out
    non-finite; the other rows stay within the bound; clean inputs count nothing."""
    c = synth.moe_case(8, 64, 256, T, 2, seed=50 + T)
    B.w4_range_events(reset=True)
    clean, _ = _moe_run(c)
    assert B.w4_range_events(reset=True) == 0
    c2 = dict(c, x=c["x"].copy())
    c2["x"][1, 7] = 1.0e5
    got, _ = _moe_run(c2)
    assert B.w4_range_events(reset=True) >= 1
    top_k = c["top_k"]
    assert not np.isfinite(got[top_k * 1:top_k * 2]).any()
    keep = np.setdiff1d(np.arange(T * top_k), np.arange(top_k, 2 * top_k))
    assert np.array_equal(got[keep], clean[keep])


# ---------------------------------------------------------------- fused SwiGLU routed mat-vec
def _swiglu_run(c, ids=None, bad=False):
    ids = c["ids"] if ids is None else ids
    bad_t = torch.zeros(1, dtype=torch.int32, device=DEV) if bad else None
    out = B.qmm_id_swiglu_q4_0(_t(c["gate"]), _t(c["up"]), _t(c["w"]), _t(ids.view(np.int32)), c["n_tokens"],
                               c["top_k"], c["N"], c["K"], c["n_experts"], c["expert_stride"], bad_ids=bad_t)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), (None if bad_t is None else int(bad_t.item()))


def _max_act(c):
    g, u = c["gate"].astype(np.float64), c["up"].astype(np.float64)
    return float(np.abs(g / (1 + np.exp(-g)) * u).max())


def test_qmm_id_swiglu_q4_0_range_event():
    c = synth.moe_swiglu_case(8, 64, 256, 2, 2, seed=60)
    B.w4_range_events(reset=True)
    _swiglu_run(c)
    assert B.w4_range_events(reset=True) == 0
    c2 = dict(c, gate=c["gate"].copy(), up=c["up"].copy())
    c2["gate"][1, 3] = 400.0
    c2["up"][1, 3] = 400.0      # silu(400) * 400 = 160000: beyond binary16
    got, _ = _swiglu_run(c2)
    assert B.w4_range_events(reset=True) >= 1
    assert not np.isfinite(got[1]).any()


@pytest.mark.parametrize("E,N,K,T,top_k", [
    (64, 1408, 2048, 1, 8),  # one decode token on the MoE workload's experts
    (8, 200, 320, 9, 3),     # ragged chunk, N not a multiple of the 32-row tile
    (6, 33, 96, 4, 1),       # odd block count (realigned spans), a 1-row last tile
    (5, 64, 8192, 2, 3),     # 4 chunks, the most the route takes
    (16, 96, 256, 32, 8),    # 256 routed rows, experts shared between tokens
])
def test_qmm_id_swiglu_q4_0(E, N, K, T, top_k):
    c = synth.moe_swiglu_case(E, N, K, T, top_k, seed=E + N + T)
    got, bad = _swiglu_run(c, bad=True)
    acc, _ = oracle.moe_swiglu_q4_0(c["gate"], c["up"], c["w"], c["ids"], T * top_k, N, K, E, c["expert_stride"])
    _assert_within(got, acc, K, _max_act(c), _max_d(c), f"swiglu E={E} N={N} K={K} T={T}")
    assert bad == 0


def test_qmm_id_swiglu_q4_0_odd_ids_and_saturated_gates():
    c = synth.moe_swiglu_case(4, 32, 64, 5, 3, seed=41)
    c["gate"][0, :6] = [-200.0, 200.0, -88.0, 88.0, -1e-30, 0.0]   # silu: -0, 200, ~0, 88, ~0, 0
    ids = c["ids"].copy()
    ids[1] = ids[0]          # the same expert twice for token 0 (different gate/up rows)
    ids[4] = 9               # no such expert
    ids[10] = 0xFFFFFFFF
    got, bad = _swiglu_run(c, ids, bad=True)
    acc, _ = oracle.moe_swiglu_q4_0(c["gate"], c["up"], c["w"], ids, 15, 32, 64, 4, c["expert_stride"])
    _assert_within(got, acc, 64, _max_act(c), _max_d(c), "swiglu odd ids")
    assert np.all(got[4] == 0) and np.all(got[10] == 0) and bad == 2
    got2, none = _swiglu_run(c, ids, bad=False)        # no count requested
    assert none is None and np.array_equal(got2, got)


# ---------------------------------------------------------------- lookup codebook, single precision
def test_qmm_lut4_f32_worked_example_from_the_page():
    # The page's unit test, exactly: every value is a dyadic rational, so the
    # f32 result must equal the printed fractions bit for bit, in both layouts.
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lut4_worked_example.json")))
    book = [i * i / 32.0 for i in range(16)]
    rows, cols, block = g["rows"], g["cols"], g["block"]
    for case in g["cases"]:
        packed = torch.full((g["packed_len"],), case["byte"], dtype=torch.uint8, device=DEV)
        scales = torch.tensor([case["scale"]], dtype=torch.float32, device=DEV)
        for transpose, key in ((0, "non_transposed"), (1, "transposed")):
            K, N = (cols, rows) if transpose else (rows, cols)
            x = torch.full((g["x_rows"], K), g["x_value"], dtype=torch.float32, device=DEV)
            y = B.qmm_lut4_f32(x, packed, scales, book, N, block, transpose=transpose).cpu().numpy()
            want = np.array([num / den for num, den in case[key]], np.float32)
            for r in range(g["x_rows"]):
                assert np.array_equal(y[r], want), (case["byte"], key, y[r], want)


def _lut_f32_case(M, K, N, block, transpose, seed):
    rng = np.random.default_rng(seed)
    count = N * K
    packed = rng.integers(0, 256, (count + 1) // 2, dtype=np.uint16).astype(np.uint8)
    scales = rng.uniform(0.01, 0.05, -(-count // block)).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    book = synth.normal_codebook()
    return x, packed, scales, book


@pytest.mark.parametrize("M,K,N,block,transpose", [
    (1, 4096, 11008, 64, 1),     # one row on the LUT workload's weights, [N, K]
    (4, 4096, 11008, 64, 0),     # four rows, the [K, N] layout
    (3, 100, 70, 6, 1),          # odd sizes: blocks straddle rows, a partial 64-lane step
    (3, 100, 70, 6, 0),
    (7, 33, 130, 2, 0),          # 3 chunks of 64 columns, K not a multiple of the 16 wavefronts
    (130, 48, 20, 16, 1),        # more than 128 rows: 33 row groups of 4
    (2, 5000, 40, 10, 0),        # 16 wavefronts over K = 5000 with blocks across rows
    (5, 520, 72, 8, 1),          # aligned [N, K] form: 65 groups of 8 (a partial 64-lane step)
    (3, 960, 40, 24, 1),         # aligned [N, K], block / 8 = 3 (not a power of two), a partial step
    (2, 1536, 48, 64, 1),        # aligned [N, K]: 3 full steps (a pair and an odd last one)
    (6, 72, 260, 4, 0),          # aligned [K, N] form: 3 column groups of 128, the last partial
    (1, 4096, 11008, 64, 0),     # one row, [K, N], the LUT workload's weights
    # [K, N] dword form (block % 8 == 0, N % block == 0): 64-column groups, 128-row chunks
    (5, 1000, 72, 8, 0),         # a partial last group, K not a multiple of the chunk, 2 row groups
    (9, 300, 4128, 32, 0),       # 65 groups: the XCD numbering's unused workgroups
    (3, 17, 64, 64, 0),          # one chunk: only the first wavefront has rows
    (4, 3000, 128, 64, 0),       # 24 chunks over 16 wavefronts (2 each for 12, none for 4)
    (2, 2304, 11008, 16, 0),     # 18 chunks over 16 wavefronts (2 each for 9)
])
def test_qmm_lut4_f32(M, K, N, block, transpose):
    x, packed, scales, book = _lut_f32_case(M, K, N, block, transpose, seed=M + K + N)
    y = B.qmm_lut4_f32(_t(x), _t(packed), _t(scales), book, N, block, transpose=transpose).cpu().numpy()
    acc, _ = oracle.lut4_f32(x, packed, scales, book, M, K, N, block, bool(transpose))
    _assert_within(y.astype(np.float64), acc, K, float(np.abs(x).max()), float(np.abs(scales).max()),
                   f"lut f32 M={M} K={K} N={N} block={block} t={transpose}")


@pytest.mark.parametrize("transpose", [0, 1])
def test_qmm_lut4_f32_compensated_sum(transpose):
    # Long K with every term positive (positive codebook and x), where a plain
    # f32 running sum gathers rounding error ~ 2^-24 sqrt(K / 3) of the total
    # (about 4e-6 here): every output stays within 1e-6 of it.
    M, K, N, block = 2, 16384, 64, 64
    x, packed, scales, book = _lut_f32_case(M, K, N, block, transpose, seed=3)
    x = np.abs(x) + 1.0
    book = np.abs(book) + np.float32(0.1)
    y = B.qmm_lut4_f32(_t(x), _t(packed), _t(scales), book, N, block, transpose=transpose).cpu().numpy()
    acc, _ = oracle.lut4_f32(x, packed, scales, book, M, K, N, block, bool(transpose))
    rows, cols = (N, K) if transpose else (K, N)
    W = oracle.lut_decode(packed, scales, book, rows, cols, block, False).astype(np.float64)
    Wt = W if transpose else W.T
    mag = np.abs(x.astype(np.float64)) @ np.abs(Wt).T
    assert np.all(np.abs(y - acc) <= 1e-6 * mag)
