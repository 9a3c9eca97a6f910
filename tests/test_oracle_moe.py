"""Pins of the expert-routed GGML Q4_0 oracle (mlx-native MoE page).

The page states the contraction (module doc) but not the Q4_0 byte layout;
the oracle reads the published GGML block (18 bytes: little-endian fp16 d, then
16 bytes whose low nibbles are elements 0..15 and high nibbles 16..31,
value = (q - 8) * d). A hand-built block pins that reading; exact integer
products, brute force in rationals and routing reductions pin the rest.
"""
from fractions import Fraction

import numpy as np

import oracle
from weight_only_bit_w4_amd import synth


def _block(d_f16_bits: int, qs) -> np.ndarray:
    return np.array([d_f16_bits & 0xFF, d_f16_bits >> 8] + list(qs), np.uint8)


def test_hand_built_block():
    qs = [(i & 15) | ((15 - i) << 4) for i in range(16)]
    blk = _block(0x3800, qs)                         # d = 0.5
    q, d = oracle.unpack_q4_0(blk, 1, 32)
    assert d[0, 0] == 0.5
    assert q[0, :16].tolist() == list(range(16))
    assert q[0, 16:].tolist() == [15 - i for i in range(16)]
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0      # picks element 0: (0 - 8) * 0.5
    x[0, 31] = 2.0     # picks element 31: q = 15 - 15 = 0 -> (0 - 8) * 0.5 * 2
    acc, out = oracle.moe_q4_0(x, blk, np.array([0], np.uint32), 1, 1, 1, 32, 1, 18)
    assert acc[0, 0] == -4.0 - 8.0 and out[0, 0] == -12.0


def test_exact_integer_when_scale_one():
    rng = np.random.default_rng(0)
    E, N, K, T, top_k = 3, 5, 64, 4, 2
    qs = rng.integers(0, 256, size=(E, N, K // 32, 16), dtype=np.uint16).astype(np.uint8)
    blocks = np.concatenate([np.broadcast_to(np.array([0x00, 0x3C], np.uint8), (E, N, K // 32, 2)), qs],
                            axis=3)
    w = blocks.reshape(-1)
    xi = rng.integers(-3, 4, size=(T, K))
    ids = np.array([0, 2, 1, 0, 2, 1, 1, 2], np.uint32)
    acc, out = oracle.moe_q4_0(xi.astype(np.float32), w, ids, T, top_k, N, K, E, N * (K // 32) * 18)
    lo = (qs & 15).astype(np.int64)
    hi = (qs >> 4).astype(np.int64)
    Wq = np.concatenate([lo, hi], axis=3).reshape(E, N, K) - 8  # per block: 16 low then 16 high
    for r in range(T * top_k):
        e, t = ids[r], r // top_k
        assert np.array_equal(acc[r], (Wq[e] @ xi[t]).astype(np.float64))
    assert np.array_equal(out, acc.astype(np.float32))


def test_brute_force_rational_tiny():
    c = synth.moe_case(4, 8, 64, 3, 2, seed=1)
    acc, out = oracle.moe_q4_0(c["x"], c["w"], c["ids"], 3, 2, 8, 64, 4, c["expert_stride"])
    wb = c["w"].reshape(4, 8, 2, 18)
    for r in range(6):
        e, t = int(c["ids"][r]), r // 2
        for n in range(8):
            terms = []
            for k in range(64):
                blk = wb[e, n, k // 32]
                d = Fraction(float(np.frombuffer(blk[0:2].tobytes(), "<f2")[0]))
                i = k % 32
                q = (blk[2 + i] & 15) if i < 16 else (blk[2 + i - 16] >> 4)
                terms.append(Fraction(float(c["x"][t, k])) * (int(q) - 8) * d)
            exact = sum(terms)
            assert abs(acc[r, n] - float(exact)) <= 64 * 2.0**-53 * float(sum(abs(v) for v in terms))


def test_top1_constant_id_is_dense_and_token_permutation():
    c = synth.moe_case(3, 16, 64, 5, 1, seed=2)
    stride = c["expert_stride"]
    for e in range(3):
        ids = np.full(5, e, np.uint32)
        acc, _ = oracle.moe_q4_0(c["x"], c["w"], ids, 5, 1, 16, 64, 3, stride)
        q, d = oracle.unpack_q4_0(c["w"][e * stride:(e + 1) * stride], 16, 64)
        Wd = (q.astype(np.float64) - 8) * np.repeat(d, 32, axis=1)
        assert np.allclose(acc, c["x"].astype(np.float64) @ Wd.T, rtol=0, atol=1e-12)
    c = synth.moe_case(6, 16, 64, 7, 3, seed=3)
    acc, _ = oracle.moe_q4_0(c["x"], c["w"], c["ids"], 7, 3, 16, 64, 6, c["expert_stride"])
    perm = np.random.default_rng(4).permutation(7)
    ids_p = c["ids"].reshape(7, 3)[perm].reshape(-1)
    accp, _ = oracle.moe_q4_0(c["x"][perm], c["w"], ids_p, 7, 3, 16, 64, 6, c["expert_stride"])
    assert np.array_equal(accp.reshape(7, 3, 16), acc.reshape(7, 3, 16)[perm])


def test_expert_stride_padding_and_out_of_range_ids():
    c = synth.moe_case(2, 4, 32, 2, 2, seed=5)
    row = 18
    per_expert = 4 * row
    pad = 40
    w = c["w"].reshape(2, per_expert)
    wp = np.zeros((2, per_expert + pad), np.uint8)
    wp[:, :per_expert] = w
    wp[:, per_expert:] = 0xFF
    acc, _ = oracle.moe_q4_0(c["x"], c["w"], c["ids"], 2, 2, 4, 32, 2, per_expert)
    accp, _ = oracle.moe_q4_0(c["x"], wp.reshape(-1), c["ids"], 2, 2, 4, 32, 2, per_expert + pad)
    assert np.array_equal(acc, accp)
    ids = c["ids"].copy()
    ids[1] = 7
    acco, _ = oracle.moe_q4_0(c["x"], c["w"], ids, 2, 2, 4, 32, 2, per_expert)
    assert np.all(acco[1] == 0) and np.array_equal(np.delete(acco, 1, 0), np.delete(acc, 1, 0))


def test_dequant_round_trip_bound():
    # our own Q4_0 quantizer: d = absmax / 7, q = round(w/d) + 8 (stays inside 0..15)
    rng = np.random.default_rng(6)
    Wt = rng.standard_normal((4, 64)).astype(np.float32) * 0.05
    blocks = []
    for n in range(4):
        for j in range(2):
            v = Wt[n, 32 * j:32 * j + 32]
            d = np.float16(np.abs(v).max() / 7)
            q = np.clip(np.round(v / np.float32(d)) + 8, 0, 15).astype(np.uint8)
            qs = (q[:16] | (q[16:] << 4)).astype(np.uint8)
            blocks.append(_block(int(np.array(d).view(np.uint16)), qs))
    w = np.concatenate(blocks)
    q, d = oracle.unpack_q4_0(w, 4, 64)
    deq = (q.astype(np.float32) - 8) * np.repeat(d, 32, axis=1)
    assert np.all(np.abs(deq - Wt) <= np.repeat(d, 32, axis=1) / 2 + 1e-7)


# ---------------------------------------------------------------- fused SwiGLU routed mat-vec
# The page's fused form (quantized_matmul_id_swiglu_q4_0 doc):
# out[r][n] = sum_k dequant(W[ids[r]][n][k]) * silu(gate[r][k]) * up[r][k],
# gate and up per routed row, silu(g) = g / (1 + e^-g).

def test_swiglu_closed_form_gate_values():
    # One weight row whose only nonzero contribution is element 0 (all other
    # gates are 0, and silu(0) = 0): out = silu(g) * up * (q - 8) * d with
    # silu(ln 3) = 3/4 ln 3 and silu(-ln 3) = -1/4 ln 3 (a flipped exponent
    # sign would give 1/4 and -3/4).
    qs = [0x0A] + [0x88] * 15                           # element 0: q = 10 -> +2; element 16: q = 0 -> -8
    blk = _block(0x3800, qs)                            # d = 0.5
    for g, silu_exact in [(np.log(3.0), 0.75 * np.log(3.0)), (-np.log(3.0), -0.25 * np.log(3.0)), (0.0, 0.0)]:
        gate = np.zeros((1, 32), np.float32)
        up = np.zeros((1, 32), np.float32)
        gate[0, 0] = np.float32(g)
        up[0, 0] = 2.0
        acc, _ = oracle.moe_swiglu_q4_0(gate, up, blk, np.array([0], np.uint32), 1, 1, 32, 1, 18)
        # The input is g rounded to f32: correct to first order with silu'(g) = s + g s (1 - s), s = sigmoid(g).
        sg = 1.0 / (1.0 + np.exp(-g))
        silu_in = silu_exact + (sg + g * sg * (1.0 - sg)) * (float(np.float32(g)) - g)
        expect = silu_in * 2.0 * 2 * 0.5                        # up * (q - 8) * d
        assert abs(acc[0, 0] - expect) <= 1e-12 * max(1.0, abs(expect)), (g, acc[0, 0], expect)


def test_swiglu_odd_part_is_the_plain_product():
    # silu(g) - silu(-g) = g exactly, so out(gate) - out(-gate) equals the
    # unfused routed product with x = gate * up (one slot per token).
    c = synth.moe_case(3, 12, 64, 6, 1, seed=7)
    rng = np.random.default_rng(8)
    gate = rng.standard_normal((6, 64)).astype(np.float32) * 2
    up = rng.standard_normal((6, 64)).astype(np.float32)
    a_pos, _ = oracle.moe_swiglu_q4_0(gate, up, c["w"], c["ids"], 6, 12, 64, 3, c["expert_stride"])
    a_neg, _ = oracle.moe_swiglu_q4_0(-gate, up, c["w"], c["ids"], 6, 12, 64, 3, c["expert_stride"])
    x = gate.astype(np.float64) * up.astype(np.float64)          # exact in f64; round to f32 for the
    acc_x, _ = oracle.moe_q4_0(x.astype(np.float32), c["w"], c["ids"], 6, 1, 12, 64, 3, c["expert_stride"])
    # f32 input of the unfused routine: its products are off by at most 2^-24 relative each
    bound = 1e-6 * np.abs(acc_x).max() + 1e-9
    assert np.all(np.abs((a_pos - a_neg) - acc_x) <= bound)


def test_swiglu_brute_force_and_degenerate_inputs():
    c = synth.moe_case(4, 5, 64, 3, 2, seed=9)
    rows = 6
    rng = np.random.default_rng(10)
    gate = (rng.standard_normal((rows, 64)) * 3).astype(np.float32)
    gate[0, :4] = [-200.0, 200.0, -1e-30, 88.0]                  # saturated and tiny gates
    up = rng.standard_normal((rows, 64)).astype(np.float32)
    ids = c["ids"].copy()
    ids[3] = 11                                                   # no such expert: zero row
    acc, out = oracle.moe_swiglu_q4_0(gate, up, c["w"], ids, rows, 5, 64, 4, c["expert_stride"])
    wb = c["w"].reshape(4, 5, 2, 18)
    for r in range(rows):
        e = int(ids[r])
        for n in range(5):
            if e >= 4:
                assert acc[r, n] == 0.0
                continue
            s = 0.0
            for k in range(64):
                blk = wb[e, n, k // 32]
                d = float(np.frombuffer(blk[0:2].tobytes(), "<f2")[0])
                i = k % 32
                q = int(blk[2 + i] & 15) if i < 16 else int(blk[2 + i - 16] >> 4)
                g = float(gate[r, k])
                sig = 1.0 / (1.0 + np.exp(-g)) if g >= 0 else np.exp(g) / (1.0 + np.exp(g))
                s += g * sig * float(up[r, k]) * (q - 8) * d
            assert abs(acc[r, n] - s) <= 1e-12 * (1 + abs(s))
    assert np.array_equal(out, acc.astype(np.float32))
    zero, _ = oracle.moe_swiglu_q4_0(gate, np.zeros_like(up), c["w"], c["ids"], rows, 5, 64, 4, c["expert_stride"])
    assert np.all(zero == 0.0)


# ---------------------------------------------------------------- point form
def test_points_equal_exact_integers_with_several_slots_and_a_bad_id():
    """moe_q4_0_points (the reference for sampled checks at the MoE workload's size) against
    exact integer arithmetic: d = 1, integer x, so every routed row must equal
    sum_k x[r // top_k][k] * (q - 8) of expert ids[r]. n_tokens != top_k, so taking the
    token as r % top_k (or the slot as the expert) gives different numbers; one id is out
    of range and must give 0."""
    rng = np.random.default_rng(7)
    E, N, K, T, top_k = 5, 6, 96, 4, 3
    qs = rng.integers(0, 256, size=(E, N, K // 32, 16), dtype=np.uint16).astype(np.uint8)
    d_one = np.broadcast_to(np.array([0x00, 0x3C], np.uint8), (E, N, K // 32, 2))
    w = np.concatenate([d_one, qs], axis=3).reshape(-1)
    xi = rng.integers(-3, 4, size=(T, K))
    ids = rng.integers(0, E, size=T * top_k).astype(np.uint32)
    ids[4] = E + 2                                     # out of range
    lo = (qs & 15).astype(np.int64)
    hi = (qs >> 4).astype(np.int64)
    Wq = np.concatenate([lo, hi], axis=3).reshape(E, N, K) - 8
    rs = np.repeat(np.arange(T * top_k), N)
    ns = np.tile(np.arange(N), T * top_k)
    pick = rng.permutation(rs.size)[:40]
    rs, ns = np.concatenate([rs[pick], [4, 4]]), np.concatenate([ns[pick], [0, N - 1]])
    acc = oracle.moe_q4_0_points(xi.astype(np.float32), w, ids, top_k, K, E, N * (K // 32) * 18, rs, ns)
    for i, (r, n) in enumerate(zip(rs, ns)):
        e, t = int(ids[r]), int(r) // top_k
        want = 0 if e >= E else int(Wq[e, n] @ xi[t])
        assert acc[i] == float(want), (r, n)


def test_points_match_the_full_routine_on_random_blocks():
    c = synth.moe_case(6, 16, 64, 5, 3, seed=8)
    ids = c["ids"].copy()
    ids[7] = 99
    acc, _ = oracle.moe_q4_0(c["x"], c["w"], ids, 5, 3, 16, 64, 6, c["expert_stride"])
    rng = np.random.default_rng(9)
    rs = rng.integers(0, 15, 60)
    ns = rng.integers(0, 16, 60)
    pa = oracle.moe_q4_0_points(c["x"], c["w"], ids, 3, 64, 6, c["expert_stride"], rs, ns)
    assert np.array_equal(pa, acc[rs, ns])
