"""ctypes binding for libw4mi.so (include/w4mi.h), argument marshalling only.

Every function has the name of the C entry point it calls. Tensors are
torch-ROCm device tensors, contiguous, with the dtypes the header states (the
16-bit float formats may be passed as torch.bfloat16 / torch.float16 or as
their raw int16 bits; uint32 words as int32). Work is enqueued on torch's
current stream of the tensors' device. There is no fallback: when the library
is missing the first call raises, and a non-OK status raises W4Error.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4mi.so")

W4_OK, W4_EINVAL, W4_EUNSUPPORTED, W4_ELAUNCH = 0, 1, 2, 3
W4_ID_SCRATCH_BAD_IDS = 0


class W4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"w4mi status {status}: {message}")
        self.status = status


class IdParams(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_uint32),
        ("top_k", ctypes.c_uint32),
        ("n", ctypes.c_uint32),
        ("k", ctypes.c_uint32),
        ("n_experts", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
        ("expert_stride", ctypes.c_uint64),
        ("x_bytes", ctypes.c_uint64),
        ("w_bytes", ctypes.c_uint64),
        ("ids_bytes", ctypes.c_uint64),
        ("out_bytes", ctypes.c_uint64),
    ]


# Exported symbols, as declared in include/w4mi.h.
_P, _I64, _I32, _U32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
SIGNATURES = {
    "w4_last_error": ([], ctypes.c_char_p),
    "w4_version": ([], ctypes.c_char_p),
    "qmm_affine4": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P], ctypes.c_int),
    "qmv_affine4": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P], ctypes.c_int),
    "qmm_lut4": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P], ctypes.c_int),
    "qmm_lut4_f32": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P], ctypes.c_int),
    "qmm_id_q4_0_scratch_bytes": ([_U32, _U32, _U32, _U32], _SZ),
    "qmm_id_q4_0": ([_P, _P, _P, _P, ctypes.POINTER(IdParams), _P, _SZ, _P], ctypes.c_int),
    "qmm_id_swiglu_q4_0": ([_P, _P, _P, _P, _P, ctypes.POINTER(IdParams), _P, _P], ctypes.c_int),
    "qmm_id_q4_0_noalloc": ([_P, _P, _P, _P, ctypes.POINTER(IdParams), _P, _P], ctypes.c_int),
    "w4_check_affine": ([_I64, _I64, _I64, _I32, _I32, _I32], ctypes.c_int),
    "w4_check_lut": ([_I64, _I64, _I64, _I32, _I32], ctypes.c_int),
    "w4_check_lut_f32": ([_I64, _I64, _I64, _I32, _I32], ctypes.c_int),
    "w4_check_id": ([ctypes.POINTER(IdParams), _SZ], ctypes.c_int),
    "w4_check_id_swiglu": ([ctypes.POINTER(IdParams)], ctypes.c_int),
    "w4_unpack_affine": ([_P, _P, _I64, _I64, _P], ctypes.c_int),
    "w4_unpack_lut": ([_P, _P, _I64, _P], ctypes.c_int),
    "w4_unpack_q4_0": ([_P, _P, _P, _I64, _I64, _P], ctypes.c_int),
    "w4_range_events": ([_P, _I32], ctypes.c_int),
    "w4_ceiling_stream_read": ([_P, ctypes.c_uint64, _P, _P], ctypes.c_int),
    "w4_ceiling_mfma": ([_P, _I32, _P], ctypes.c_int),
}

_lock = threading.Lock()
_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m weight_only_bit_w4_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.argtypes = args
                fn.restype = res
            _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != W4_OK:
        raise W4Error(status, lib().w4_last_error().decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _shape(t, name: str, shape) -> None:
    """Raises unless tensor t has exactly `shape` (checked before any device work)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _numel_at_least(t, name: str, count: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.numel() < count:
        raise ValueError(f"{name} holds {t.numel()} elements, expected at least {count}")


def _same_device(ref: torch.Tensor, **tensors) -> None:
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, the call runs on {ref.device}")


def _dev(t: torch.Tensor, name: str, dtypes) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


BF16 = (torch.bfloat16, torch.int16)
F16 = (torch.float16, torch.int16)
U32 = (torch.int32,)
U8 = (torch.uint8,)
F32 = (torch.float32,)


def version() -> str:
    return lib().w4_version().decode()


# ---------------------------------------------------------------- affine INT4
def _affine(fn_name, w, scales, biases, x, y, group_size, bits):
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x must be [M, K] and w [N, K/8]")
    M, K = x.shape
    N = w.shape[0]
    if group_size > 0 and K % group_size == 0 and K % 8 == 0:
        _shape(w, "w", (N, K // 8))
        _shape(scales, "scales", (N, K // group_size))
        _shape(biases, "biases", (N, K // group_size))
    if y is not None:
        _shape(y, "y", (M, N))
    _same_device(x, w=w, scales=scales, biases=biases, y=y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    fn = getattr(lib(), fn_name)
    _check(fn(_dev(w, "w", U32), _dev(scales, "scales", BF16), _dev(biases, "biases", BF16), _dev(x, "x", BF16),
              _dev(y, "y", BF16), M, K, N, group_size, bits, _stream(x)))
    return y


def qmm_affine4(w, scales, biases, x, y=None, group_size: int = 32, bits: int = 4):
    """y [M, N] bf16 = x [M, K] bf16 . (q * scale + bias)^T, M > 1."""
    return _affine("qmm_affine4", w, scales, biases, x, y, group_size, bits)


def qmv_affine4(w, scales, biases, x, y=None, group_size: int = 32, bits: int = 4):
    """y [1, N] bf16 = x [1, K] bf16 . (q * scale + bias)^T (decode GEMV)."""
    return _affine("qmv_affine4", w, scales, biases, x, y, group_size, bits)


# ---------------------------------------------------------------- lookup codebook
def _lut_shapes(x, packed, scales, book, N, block, y):
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    if len(book) != 16:
        raise ValueError(f"book holds {len(book)} values, expected 16")
    if N > 0 and K > 0 and block > 0:
        count = N * K
        _numel_at_least(packed, "packed", (count + 1) // 2)
        _numel_at_least(scales, "scales", -(-count // block))
    if y is not None:
        _shape(y, "y", (M, N))
    _same_device(x, packed=packed, scales=scales, y=y)


def qmm_lut4(x, packed, scales, book, N: int, block: int, y=None, transpose: int = 1):
    """y [M, N] fp16 = x [M, K] fp16 . fp16(book[code] * scale)^T; book: 16 host floats."""
    _lut_shapes(x, packed, scales, book, N, block, y)
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    book_host = (ctypes.c_float * 16)(*[float(v) for v in book])
    _check(lib().qmm_lut4(_dev(x, "x", F16), _dev(packed, "packed", U8), _dev(scales, "scales", F16),
                          ctypes.cast(book_host, ctypes.c_void_p), _dev(y, "y", F16), M, K, N, block, transpose,
                          _stream(x)))
    return y


def qmm_lut4_f32(x, packed, scales, book, N: int, block: int, y=None, transpose: int = 1):
    """y [M, N] f32 = x [M, K] f32 . W, W = book[code] * scale (f32, unrounded); W is [N, K]
    when transpose else [K, N]; book: 16 host floats."""
    _lut_shapes(x, packed, scales, book, N, block, y)
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    book_host = (ctypes.c_float * 16)(*[float(v) for v in book])
    _check(lib().qmm_lut4_f32(_dev(x, "x", F32), _dev(packed, "packed", U8), _dev(scales, "scales", F32),
                              ctypes.cast(book_host, ctypes.c_void_p), _dev(y, "y", F32), M, K, N, block, transpose,
                              _stream(x)))
    return y


# ---------------------------------------------------------------- expert-routed Q4_0
def qmm_id_q4_0_scratch_bytes(n_experts: int, n_tokens: int, top_k: int, k: int) -> int:
    return int(lib().qmm_id_q4_0_scratch_bytes(n_experts, n_tokens, top_k, k))


def id_params(x, w, ids, out, n_tokens, top_k, n, k, n_experts, expert_stride) -> IdParams:
    return IdParams(n_tokens, top_k, n, k, n_experts, 0, expert_stride,
                    x.numel() * x.element_size(), w.numel() * w.element_size(),
                    ids.numel() * ids.element_size(), out.numel() * out.element_size())


def qmm_id_q4_0(x, w, ids, n_tokens: int, top_k: int, n: int, k: int, n_experts: int, expert_stride: int,
                out=None, scratch=None):
    """out [n_tokens*top_k, n] f32: routed rows through their experts' Q4_0 weights."""
    _same_device(x, w=w, ids=ids, out=out, scratch=scratch)
    if out is None:
        out = torch.empty((n_tokens * top_k, n), dtype=torch.float32, device=x.device)
    if scratch is None:
        scratch = torch.empty(qmm_id_q4_0_scratch_bytes(n_experts, n_tokens, top_k, k), dtype=torch.uint8,
                              device=x.device)
    p = id_params(x, w, ids, out, n_tokens, top_k, n, k, n_experts, expert_stride)
    _check(lib().qmm_id_q4_0(_dev(x, "x", F32), _dev(w, "w", U8), _dev(ids, "ids", U32), _dev(out, "out", F32),
                             ctypes.byref(p), _dev(scratch, "scratch", U8), scratch.numel(), _stream(x)))
    return out


def qmm_id_q4_0_noalloc(x, w, ids, n_tokens: int, top_k: int, n: int, k: int, n_experts: int, expert_stride: int,
                        out=None, bad_ids=None):
    """qmm_id_q4_0 with the library's fixed device scratch (no allocation in the library). out must be
    passed for a call that may not allocate at all; bad_ids: optional device int32 [1]."""
    _same_device(x, w=w, ids=ids, out=out, bad_ids=bad_ids)
    if out is None:
        out = torch.empty((n_tokens * top_k, n), dtype=torch.float32, device=x.device)
    p = id_params(x, w, ids, out, n_tokens, top_k, n, k, n_experts, expert_stride)
    bad = None if bad_ids is None else _dev(bad_ids, "bad_ids", U32)
    _check(lib().qmm_id_q4_0_noalloc(_dev(x, "x", F32), _dev(w, "w", U8), _dev(ids, "ids", U32),
                                     _dev(out, "out", F32), ctypes.byref(p), bad, _stream(x)))
    return out


def qmm_id_swiglu_q4_0(gate, up, w, ids, n_tokens: int, top_k: int, n: int, k: int, n_experts: int,
                       expert_stride: int, out=None, bad_ids=None):
    """out [n_tokens*top_k, n] f32 = dequant(W[ids[r]]) . (silu(gate[r]) * up[r]) per routed row r.
    bad_ids: optional device uint32 tensor [1] receiving the out-of-range id count."""
    if out is None:
        out = torch.empty((n_tokens * top_k, n), dtype=torch.float32, device=gate.device)
    if up.shape != gate.shape:
        raise ValueError("gate and up must have the same shape")
    _same_device(gate, up=up, w=w, ids=ids, out=out, bad_ids=bad_ids)
    p = id_params(gate, w, ids, out, n_tokens, top_k, n, k, n_experts, expert_stride)
    bad = None if bad_ids is None else _dev(bad_ids, "bad_ids", U32)
    _check(lib().qmm_id_swiglu_q4_0(_dev(gate, "gate", F32), _dev(up, "up", F32), _dev(w, "w", U8),
                                    _dev(ids, "ids", U32), _dev(out, "out", F32), ctypes.byref(p), bad,
                                    _stream(gate)))
    return out


# ---------------------------------------------------------------- host checks
def w4_check_affine(M, K, N, group_size=32, bits=4, decode=0) -> int:
    return int(lib().w4_check_affine(M, K, N, group_size, bits, decode))


def w4_check_lut(M, K, N, block, transpose=1) -> int:
    return int(lib().w4_check_lut(M, K, N, block, transpose))


def w4_check_lut_f32(M, K, N, block, transpose=1) -> int:
    return int(lib().w4_check_lut_f32(M, K, N, block, transpose))


def w4_check_id(params: IdParams, scratch_bytes: int) -> int:
    return int(lib().w4_check_id(ctypes.byref(params), scratch_bytes))


def w4_check_id_swiglu(params: IdParams) -> int:
    return int(lib().w4_check_id_swiglu(ctypes.byref(params)))


def w4_range_events(reset: bool = False) -> int:
    """Range events of qmm_affine4's binary16 routes on the current device (synchronises it)."""
    n = ctypes.c_uint32(0)
    _check(lib().w4_range_events(ctypes.byref(n), int(reset)))
    return int(n.value)


def w4_ceiling_stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Reads every byte of buf once (streaming-read ceiling); sink: device int32 [1024]."""
    _numel_at_least(sink, "sink", 1024)
    _check(lib().w4_ceiling_stream_read(_dev(buf, "buf", (buf.dtype,)), buf.numel() * buf.element_size(),
                                        _dev(sink, "sink", U32), _stream(buf)))


def w4_ceiling_mfma(sink: torch.Tensor, iters: int) -> None:
    """Back-to-back f16 matrix-core instructions on every SIMD (MFMA ceiling); sink: device int32 [1024]."""
    _numel_at_least(sink, "sink", 1024)
    _check(lib().w4_ceiling_mfma(_dev(sink, "sink", U32), iters, _stream(sink)))


def last_error() -> str:
    return lib().w4_last_error().decode()


# ---------------------------------------------------------------- unpack exports
def w4_unpack_affine(w, N: int, K: int):
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    _check(lib().w4_unpack_affine(_dev(w, "w", U32), _dev(q, "q", U8), N, K, _stream(w)))
    return q


def w4_unpack_lut(packed, count: int):
    codes = torch.empty(count, dtype=torch.uint8, device=packed.device)
    _check(lib().w4_unpack_lut(_dev(packed, "packed", U8), _dev(codes, "codes", U8), count, _stream(packed)))
    return codes


def w4_unpack_q4_0(w, rows: int, K: int):
    q = torch.empty((rows, K), dtype=torch.uint8, device=w.device)
    d = torch.empty((rows, K // 32), dtype=torch.int16, device=w.device)
    _check(lib().w4_unpack_q4_0(_dev(w, "w", U8), _dev(q, "q", U8), _dev(d, "d", (torch.int16,)), rows, K,
                                _stream(w)))
    return q, d
