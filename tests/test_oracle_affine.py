"""Pins of the affine INT4 oracle (INT4 group-32 MatMulNBits page).

Each check is independent of the oracle's own code path: nibbles by integer
division, exact integer matmul, a closed form for constant scale and zero
point, brute force in rational arithmetic, a quantize -> dequantize round trip
bound, and reductions (row independence, permutation).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from weight_only_bit_w4_amd import synth

BF16_ONE = 0x3F80


def bf16_bits(a):
    t = torch.from_numpy(np.asarray(a, np.float32).copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_value(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy()).view(torch.bfloat16).float().numpy()


def test_unpack_matches_integer_division():
    rng = np.random.default_rng(0)
    N, K = 7, 64
    w = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    q = oracle.unpack_affine(w, N, K)
    for n in range(N):
        for k in range(K):
            word = int(w[n, k // 8])
            assert q[n, k] == (word // 16 ** (k % 8)) % 16


def test_unpack_is_lsb_first():
    # the page's test packs nib j of a word at bit 4j: word = sum_j q_j * 16^j
    q = np.array([[0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15]], np.uint8)
    words = np.array([[sum(int(q[0, j]) * 16**j for j in range(8)),
                       sum(int(q[0, 8 + j]) * 16**j for j in range(8))]], np.uint32)
    assert words[0, 0] == 0x76543210 and words[0, 1] == 0xFEDCBA98
    assert np.array_equal(oracle.unpack_affine(words, 1, 16), q)


def test_exact_integer_matmul_when_scale_one_bias_zero():
    rng = np.random.default_rng(3)
    M, K, N = 5, 96, 40
    w = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    scales = np.full((N, K // 32), BF16_ONE, np.uint16)
    biases = np.zeros((N, K // 32), np.uint16)
    xi = rng.integers(-3, 4, size=(M, K))
    x = bf16_bits(xi)
    acc, y = oracle.affine(w, scales, biases, x, M, K, N)
    q = np.array([[(int(w[n, k // 8]) >> (4 * (k % 8))) & 15 for k in range(K)] for n in range(N)])
    ref = xi @ q.T
    assert np.array_equal(acc, ref.astype(np.float64))
    assert np.array_equal(y, bf16_bits(ref.astype(np.float32)))


def test_closed_form_constant_scale_and_zero_point():
    # w = s*(q - zp) for every group: y = s * (x q^T) - zp * s * sum_k x
    rng = np.random.default_rng(4)
    M, K, N = 3, 128, 24
    w = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    s_bits = bf16_bits([0.0078125])[0]           # 2^-7: q*s and zp*s are exact
    zp = 5
    b_bits = bf16_bits([-zp * 0.0078125])[0]
    scales = np.full((N, K // 32), s_bits, np.uint16)
    biases = np.full((N, K // 32), b_bits, np.uint16)
    x = bf16_bits(rng.standard_normal((M, K)))
    xv = bf16_value(x).astype(np.float64)
    acc, _ = oracle.affine(w, scales, biases, x, M, K, N)
    q = np.array([[(int(w[n, k // 8]) >> (4 * (k % 8))) & 15 for k in range(K)] for n in range(N)],
                 np.float64)
    ref = 0.0078125 * (xv @ q.T) - zp * 0.0078125 * xv.sum(axis=1, keepdims=True)
    bound = 4 * K * np.finfo(np.float64).eps * (np.abs(xv) @ np.abs(q.T * 0.0078125 - zp * 0.0078125))
    assert np.all(np.abs(acc - ref) <= bound)


def _exact_weight(q, s_bits, b_bits):
    s = Fraction(float(bf16_value([s_bits])[0]))
    b = Fraction(float(bf16_value([b_bits])[0]))
    exact = q * s + b                         # needs < 53 bits: float() is exact
    return Fraction(float(np.float32(float(exact))))  # one rounding to f32, as the page's host reference


def test_brute_force_rational_tiny():
    case = synth.affine_case(2, 64, 32, seed=5)
    M, K, N = 2, 64, 32
    acc, y = oracle.affine(case["w"], case["scales"], case["biases"], case["x"], M, K, N)
    xv = bf16_value(case["x"])
    for m in range(M):
        for n in range(N):
            terms = []
            for k in range(K):
                q = (int(case["w"][n, k // 8]) >> (4 * (k % 8))) & 15
                g = k // 32
                wv = _exact_weight(q, case["scales"][n, g], case["biases"][n, g])
                terms.append(Fraction(float(xv[m, k])) * wv)
            exact = sum(terms)
            bound = K * 2.0**-53 * float(sum(abs(t) for t in terms))
            assert abs(acc[m, n] - float(exact)) <= bound
            # the output is the bf16 RNE of the f32 rounding of the exact sum (no sum here
            # lies within the fp64 error of a rounding boundary, so the double rounding agrees)
            assert y[m, n] == bf16_bits([np.float32(float(exact))])[0]


def test_quantize_dequantize_round_trip_bound():
    # our own min-max quantizer (the pages define none): s = (max-min)/15, zp = round(-min/s)
    rng = np.random.default_rng(6)
    N, K = 16, 256
    W = rng.standard_normal((N, K)).astype(np.float32) * 0.1
    G = K // 32
    Wg = W.reshape(N, G, 32)
    lo, hi = Wg.min(axis=2), Wg.max(axis=2)
    s = ((hi - lo) / 15).astype(np.float32)
    zp = np.clip(np.round(-lo / s), 0, 15)
    q = np.clip(np.round(Wg / s[..., None] + zp[..., None]), 0, 15).astype(np.uint32)
    words = np.zeros((N, K // 8), np.uint32)
    qf = q.reshape(N, K)
    for j in range(8):
        words |= (qf[:, j::8] << (4 * j)).astype(np.uint32)
    s_bits, b_bits = bf16_bits(s), bf16_bits(-zp * s)
    deq = oracle.dequant_affine(words, s_bits, b_bits, N, K)
    s_b = bf16_value(s_bits)
    b_b = bf16_value(b_bits)
    # |deq - w| <= s/2 (quantization) + 15*|s - s_bf16| + |b - b_bf16| (bf16 storage of s, b) + f32 rounding
    err_s = np.abs(s - s_b)
    err_b = np.abs(-zp * s - b_b)
    bound = s / 2 + 15 * err_s + err_b + 1e-6
    assert np.all(np.abs(deq.reshape(N, G, 32) - Wg) <= bound[..., None])


def test_rows_independent_and_permutation():
    case = synth.affine_case(6, 128, 64, seed=7)
    M, K, N = 6, 128, 64
    acc, y = oracle.affine(case["w"], case["scales"], case["biases"], case["x"], M, K, N)
    # a single row (the decode GEMV shape) is the same computation
    acc1, y1 = oracle.affine(case["w"], case["scales"], case["biases"], case["x"][3:4], 1, K, N)
    assert np.array_equal(acc1[0], acc[3]) and np.array_equal(y1[0], y[3])
    perm = np.random.default_rng(8).permutation(M)
    accp, _ = oracle.affine(case["w"], case["scales"], case["biases"], case["x"][perm], M, K, N)
    assert np.array_equal(accp, acc[perm])
    # points entry agrees with the full one
    ms = np.array([0, 5, 2]); ns = np.array([63, 0, 17])
    pa, py = oracle.affine_points(case["w"], case["scales"], case["biases"], case["x"], K, ms, ns)
    assert np.array_equal(pa, acc[ms, ns]) and np.array_equal(py, y[ms, ns])


@pytest.mark.parametrize("flip", ["scale", "bias", "nibble"])
def test_single_operand_change_moves_only_its_outputs(flip):
    case = synth.affine_case(2, 64, 32, seed=9)
    M, K, N = 2, 64, 32
    acc, _ = oracle.affine(case["w"], case["scales"], case["biases"], case["x"], M, K, N)
    c = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in case.items()}
    n, g = 11, 1
    if flip == "scale":
        c["scales"][n, g] = bf16_bits([0.5])[0]
    elif flip == "bias":
        c["biases"][n, g] = bf16_bits([0.25])[0]
    else:
        c["w"][n, 4 * g] ^= 0xF
    acc2, _ = oracle.affine(c["w"], c["scales"], c["biases"], c["x"], M, K, N)
    changed = np.any(acc2 != acc, axis=0)
    assert changed[n] and changed.sum() == 1
