"""CPU oracle for y = x . dequant(W)^T with 4-bit weights (affine INT4, lookup
codebook, expert-routed GGML Q4_0).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The HIP library never
calls it and shares no code with it; see ``oracle.c`` for the conventions and
the passages of the pages each function follows.

Every function takes and returns numpy arrays holding the stored bit patterns
(bf16 / fp16 as ``uint16``), and computes through the C routines in
``oracle.c`` (fp64 accumulation, the file's own 16-bit float conversions).

Parity status: every function here is pinned by tests in ``tests/test_oracle_*``
(worked example of the lookup page, exact integer cases, closed forms,
brute force in rational arithmetic, round-trip bounds, reductions), except the
GGML Q4_0 byte layout, which the pages name but never define: its reading (the
published GGML block) is pinned only against hand-built blocks written from
that reading.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with the host compiler (gcc, OpenMP, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I = ctypes.c_int64
            U = ctypes.c_uint64
            C = ctypes.c_int
            sig = {
                "w4o_bf16_to_f32_n": [P, P, I],
                "w4o_f32_to_bf16_n": [P, P, I],
                "w4o_f16_to_f32_n": [P, P, I],
                "w4o_f32_to_f16_n": [P, P, I],
                "w4o_unpack_affine": [P, I, I, P],
                "w4o_dequant_affine": [P, P, P, I, I, I, P],
                "w4o_affine": [P, P, P, P, I, I, I, I, P, P],
                "w4o_affine_points": [P, P, P, P, I, I, P, P, I, P, P],
                "w4o_unpack_lut": [P, I, P],
                "w4o_lut_decode": [P, P, P, I, I, I, C, P],
                "w4o_lut_matmul": [P, P, I, I, I, C, P],
                "w4o_lut_points": [P, P, P, P, I, I, C, P, P, I, P],
                "w4o_unpack_q4_0": [P, I, I, P, P],
                "w4o_moe_q4_0": [P, P, P, I, I, I, I, I, U, P, P],
                "w4o_moe_q4_0_points": [P, P, P, I, I, I, U, P, P, I, P],
                "w4o_moe_swiglu_q4_0": [P, P, P, P, I, I, I, I, U, P, P],
            }
            for name, args in sig.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = None
            _lib = lib
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else the affinity mask)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    return len(os.sched_getaffinity(0))


# ---------------------------------------------------------------- conversions
def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().w4o_bf16_to_f32_n(_p(h), _p(out), h.size)
    return out


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().w4o_f32_to_bf16_n(_p(f), _p(out), f.size)
    return out


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().w4o_f16_to_f32_n(_p(h), _p(out), h.size)
    return out


def f32_to_f16(f: np.ndarray) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().w4o_f32_to_f16_n(_p(f), _p(out), f.size)
    return out


# ---------------------------------------------------------------- affine INT4
def unpack_affine(w: np.ndarray, N: int, K: int) -> np.ndarray:
    w = _c(w, np.uint32)
    assert w.size == N * K // 8
    q = np.empty((N, K), np.uint8)
    _load().w4o_unpack_affine(_p(w), N, K, _p(q))
    return q


def dequant_affine(w, scales, biases, N: int, K: int, group: int = 32) -> np.ndarray:
    w, s, b = _c(w, np.uint32), _c(scales, np.uint16), _c(biases, np.uint16)
    W = np.empty((N, K), np.float32)
    _load().w4o_dequant_affine(_p(w), _p(s), _p(b), N, K, group, _p(W))
    return W


def affine(w, scales, biases, x, M: int, K: int, N: int, group: int = 32):
    """Returns (acc fp64 [M, N], y bf16 bits [M, N])."""
    w, s, b, x = _c(w, np.uint32), _c(scales, np.uint16), _c(biases, np.uint16), _c(x, np.uint16)
    assert w.size == N * K // 8 and s.size == N * K // group and b.size == s.size and x.size == M * K
    acc = np.empty((M, N), np.float64)
    y = np.empty((M, N), np.uint16)
    _load().w4o_affine(_p(w), _p(s), _p(b), _p(x), M, K, N, group, _p(acc), _p(y))
    return acc, y


def affine_points(w, scales, biases, x, K: int, ms, ns, group: int = 32):
    """fp64 sums and bf16 outputs at the (ms[i], ns[i]) points only."""
    w, s, b, x = _c(w, np.uint32), _c(scales, np.uint16), _c(biases, np.uint16), _c(x, np.uint16)
    ms, ns = _c(ms, np.int64), _c(ns, np.int64)
    acc = np.empty(ms.size, np.float64)
    y = np.empty(ms.size, np.uint16)
    _load().w4o_affine_points(_p(w), _p(s), _p(b), _p(x), K, group, _p(ms), _p(ns), ms.size, _p(acc), _p(y))
    return acc, y


# ---------------------------------------------------------------- lookup codebook
def unpack_lut(packed: np.ndarray, count: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    assert packed.size * 2 >= count
    codes = np.empty(count, np.uint8)
    _load().w4o_unpack_lut(_p(packed), count, _p(codes))
    return codes


def lut_decode(packed, scales_f32, book, rows: int, cols: int, block: int, round_half: bool):
    packed, s, book = _c(packed, np.uint8), _c(scales_f32, np.float32), _c(book, np.float32)
    assert book.size == 16 and s.size == -(-rows * cols // block)
    W = np.empty((rows, cols), np.float32)
    _load().w4o_lut_decode(_p(packed), _p(s), _p(book), rows, cols, block, int(round_half), _p(W))
    return W


def lut_matmul(x_f32, W, M: int, K: int, N: int, transpose: bool) -> np.ndarray:
    x, W = _c(x_f32, np.float32), _c(W, np.float32)
    assert x.size == M * K and W.size == K * N
    acc = np.empty((M, N), np.float64)
    _load().w4o_lut_matmul(_p(x), _p(W), M, K, N, int(transpose), _p(acc))
    return acc


def lut4(x_f16, packed, scales_f16, book, M: int, K: int, N: int, block: int,
         transpose: bool = True, round_half: bool = True):
    """fp16 path: x fp16 [M, K], scales fp16, decoded weight rounded to fp16 when
    round_half, y fp16 [M, N]. Returns (acc fp64, y fp16 bits)."""
    rows, cols = (N, K) if transpose else (K, N)
    W = lut_decode(packed, f16_to_f32(scales_f16), book, rows, cols, block, round_half)
    acc = lut_matmul(f16_to_f32(x_f16), W, M, K, N, transpose)
    y = f32_to_f16(acc.astype(np.float32))
    return acc, y


def lut4_f32(x_f32, packed, scales_f32, book, M: int, K: int, N: int, block: int, transpose: bool = True):
    """Single-precision path: x f32, scales f32, the decoded weight not rounded,
    y f32. Returns (acc fp64 [M, N], y f32)."""
    rows, cols = (N, K) if transpose else (K, N)
    W = lut_decode(packed, scales_f32, book, rows, cols, block, False)
    acc = lut_matmul(x_f32, W, M, K, N, transpose)
    return acc, acc.astype(np.float32)


def lut4_points(x_f16, packed, scales_f16, book, K: int, block: int, ms, ns, round_half: bool = True):
    x, packed, s, book = _c(x_f16, np.uint16), _c(packed, np.uint8), _c(scales_f16, np.uint16), _c(book, np.float32)
    ms, ns = _c(ms, np.int64), _c(ns, np.int64)
    acc = np.empty(ms.size, np.float64)
    _load().w4o_lut_points(_p(x), _p(packed), _p(s), _p(book), K, block, int(round_half),
                           _p(ms), _p(ns), ms.size, _p(acc))
    return acc


# ---------------------------------------------------------------- MoE GGML Q4_0
Q4_0_QK = 32
Q4_0_BYTES = 18


def unpack_q4_0(w_bytes: np.ndarray, rows: int, K: int):
    """Codes q [rows, K] (0..15) and scales d f32 [rows, K/32] of consecutive rows."""
    w = _c(w_bytes, np.uint8)
    assert w.size >= rows * (K // Q4_0_QK) * Q4_0_BYTES
    q = np.empty((rows, K), np.uint8)
    d = np.empty((rows, K // Q4_0_QK), np.float32)
    _load().w4o_unpack_q4_0(_p(w), rows, K, _p(q), _p(d))
    return q, d


def moe_q4_0(x, w_bytes, ids, n_tokens: int, top_k: int, N: int, K: int, n_experts: int,
             expert_stride: int):
    """Returns (acc fp64 [n_tokens*top_k, N], out f32 [n_tokens*top_k, N])."""
    x, w, ids = _c(x, np.float32), _c(w_bytes, np.uint8), _c(ids, np.uint32)
    rows = n_tokens * top_k
    assert x.size == n_tokens * K and ids.size == rows
    acc = np.empty((rows, N), np.float64)
    out = np.empty((rows, N), np.float32)
    _load().w4o_moe_q4_0(_p(x), _p(w), _p(ids), n_tokens, top_k, N, K, n_experts, expert_stride,
                         _p(acc), _p(out))
    return acc, out


def moe_q4_0_points(x, w_bytes, ids, top_k: int, K: int, n_experts: int, expert_stride: int, rs, ns):
    x, w, ids = _c(x, np.float32), _c(w_bytes, np.uint8), _c(ids, np.uint32)
    rs, ns = _c(rs, np.int64), _c(ns, np.int64)
    acc = np.empty(rs.size, np.float64)
    _load().w4o_moe_q4_0_points(_p(x), _p(w), _p(ids), top_k, K, n_experts, expert_stride,
                                _p(rs), _p(ns), rs.size, _p(acc))
    return acc


def moe_swiglu_q4_0(gate, up, w_bytes, ids, rows: int, N: int, K: int, n_experts: int, expert_stride: int):
    """Fused SwiGLU routed mat-vec: returns (acc fp64 [rows, N], out f32 [rows, N]) for
    out[r][n] = sum_k dequant(W[ids[r]][n][k]) * silu(gate[r][k]) * up[r][k]."""
    gate, up = _c(gate, np.float32), _c(up, np.float32)
    w, ids = _c(w_bytes, np.uint8), _c(ids, np.uint32)
    assert gate.size == rows * K and up.size == rows * K and ids.size == rows
    acc = np.empty((rows, N), np.float64)
    out = np.empty((rows, N), np.float32)
    _load().w4o_moe_swiglu_q4_0(_p(gate), _p(up), _p(w), _p(ids), rows, N, K, n_experts, expert_stride,
                                _p(acc), _p(out))
    return acc, out


# ---------------------------------------------------------------- tolerance
def tolerance(ref: np.ndarray, K: int, max_abs_x: float, max_abs_scale: float) -> np.ndarray:
    """Per-element bound |y - ref| <= 1e-2 |ref| + 1e-2 sqrt(K) max|x| max|scale|,
    with ref the fp64 accumulator."""
    return 1e-2 * np.abs(ref) + 1e-2 * np.sqrt(K) * max_abs_x * max_abs_scale
