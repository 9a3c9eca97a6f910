"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol include/w4mi.h declares, and its argument contracts reject what the
pages' validation rejects, before any device work."""
import os
import re

import pytest

from weight_only_bit_w4_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4mi.h")


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(B.LIB_PATH):
        from weight_only_bit_w4_amd import build
        build.build(verbose=False)
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([A-Za-z_]\w*)\s*\(", text)) - {"if", "sizeof", "return"})


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"qmm_affine4", "qmv_affine4", "qmm_lut4", "qmm_id_q4_0"} <= set(names)
    lib = B.lib()
    for name in names:
        assert hasattr(lib, name), name
        assert name in B.SIGNATURES, f"binding lacks {name}"


def test_version():
    assert "gfx950" in B.version()


@pytest.mark.parametrize("args,status,needle", [
    ((4, 256, 256, 32, 4, 0), B.W4_OK, ""),
    ((1, 4096, 14336, 32, 4, 1), B.W4_OK, ""),
    ((0, 64, 64, 32, 4, 0), B.W4_OK, ""),
    ((1, 256, 256, 32, 4, 0), B.W4_EINVAL, "M > 1"),          # prefill kernel is M > 1 only
    ((2, 256, 256, 32, 4, 1), B.W4_EINVAL, "M == 1"),         # decode GEMV is M == 1 only
    ((4, 256, 256, 64, 4, 0), B.W4_EINVAL, "group_size"),
    ((4, 256, 256, 32, 8, 0), B.W4_EINVAL, "bits"),
    ((4, 250, 256, 32, 4, 0), B.W4_EINVAL, "K (250)"),
    ((4, 256, 250, 32, 4, 0), B.W4_EINVAL, "N (250)"),
    ((4, 0, 256, 32, 4, 0), B.W4_EINVAL, "K, N > 0"),
    ((-1, 64, 64, 32, 4, 0), B.W4_EINVAL, "M >= 0"),
])
def test_affine_contract(args, status, needle):
    assert B.w4_check_affine(*args) == status
    if status != B.W4_OK:
        assert needle in B.last_error()


@pytest.mark.parametrize("args,status", [
    ((512, 4096, 11008, 64, 1), B.W4_OK),
    ((0, 4096, 11008, 64, 1), B.W4_OK),
    ((5, 128, 48, 63, 1), B.W4_EINVAL),          # block must be even
    ((5, 128, 48, 0, 1), B.W4_EINVAL),
    ((5, 0, 48, 64, 1), B.W4_EINVAL),
    ((5, 128, 48, 64, 0), B.W4_OK),              # [K, N] layout (vector-ALU column kernels)
    ((5, 5, 3, 64, 0), B.W4_OK),                 # [K, N] with blocks across rows
    ((262141, 32, 32, 2, 0), B.W4_EUNSUPPORTED), # [K, N] past 4 rows x 65535 workgroups
    ((5, 96, 48, 64, 1), B.W4_EUNSUPPORTED),     # K not a multiple of the block
    ((5, 128, 48, 2, 1), B.W4_EUNSUPPORTED),     # block not a multiple of 8
])
def test_lut_contract(args, status):
    assert B.w4_check_lut(*args) == status


def _params(**kw):
    base = dict(n_tokens=128, top_k=8, n=1408, k=2048, n_experts=64, expert_stride=1408 * 64 * 18)
    base.update(kw)
    rows = base["n_tokens"] * base["top_k"]
    p = B.IdParams(base["n_tokens"], base["top_k"], base["n"], base["k"], base["n_experts"], 0,
                   base["expert_stride"], base["n_tokens"] * base["k"] * 4,
                   base["n_experts"] * base["expert_stride"], rows * 4, rows * base["n"] * 4)
    for f in ("x_bytes", "w_bytes", "ids_bytes", "out_bytes", "reserved"):
        if f in kw:
            setattr(p, f, kw[f])
    return p, B.qmm_id_q4_0_scratch_bytes(base["n_experts"], base["n_tokens"], base["top_k"], base["k"])


@pytest.mark.parametrize("kw,status,needle", [
    ({}, B.W4_OK, ""),
    ({"n_tokens": 0}, B.W4_EINVAL, "every size must be positive"),
    ({"top_k": 0}, B.W4_EINVAL, "top_k=0"),
    ({"n_experts": 0}, B.W4_EINVAL, "n_experts=0"),
    ({"k": 2047}, B.W4_EINVAL, "whole number of 32-weight"),
    ({"expert_stride": 1000}, B.W4_EINVAL, "experts are 1000 bytes apart"),
    ({"x_bytes": 16}, B.W4_EINVAL, "x holds 16 bytes"),
    ({"w_bytes": 1}, B.W4_EINVAL, "w holds 1 bytes"),
    ({"ids_bytes": 4}, B.W4_EINVAL, "ids holds 4 bytes"),
    ({"out_bytes": 4}, B.W4_EINVAL, "out holds 4 bytes"),
    ({"reserved": 1}, B.W4_EINVAL, "reserved field"),
])
def test_id_contract(kw, status, needle):
    p, scratch = _params(**kw)
    assert B.w4_check_id(p, scratch) == status
    if status != B.W4_OK:
        assert needle in B.last_error()


def test_id_scratch_too_small():
    p, scratch = _params()
    assert B.w4_check_id(p, scratch - 1) == B.W4_EINVAL
    assert "scratch" in B.last_error()


def test_id_stride_padding_counts_last_expert_only():
    # the last expert's slab need not be padded to the full stride
    p, scratch = _params(expert_stride=1408 * 64 * 18 + 64)
    p.w_bytes = 63 * (1408 * 64 * 18 + 64) + 1408 * 64 * 18
    assert B.w4_check_id(p, scratch) == B.W4_OK
    p.w_bytes -= 1
    assert B.w4_check_id(p, scratch) == B.W4_EINVAL


def _fake(addr=0x100000):
    import ctypes
    return ctypes.c_void_p(addr)


def test_affine_prefill_size_limit_is_reported_before_any_launch():
    # K past 2^21: a valid shape this library does not implement; the call
    # returns before touching the (fake) device pointers.
    lib = B.lib()
    K = (1 << 21) + 32
    st = lib.qmm_affine4(_fake(), _fake(), _fake(), _fake(), _fake(), 4, K, 256, 32, 4, None)
    assert st == B.W4_EUNSUPPORTED
    assert "2097152" in B.last_error()


def test_id_size_limit_is_reported_before_any_launch():
    lib = B.lib()
    import ctypes
    p, scratch = _params(n_tokens=1 << 20)  # n_tokens * K * 2 = 2^32 bytes of binary16 x
    st = lib.qmm_id_q4_0(_fake(), _fake(), _fake(), _fake(), ctypes.byref(p), _fake(), ctypes.c_size_t(scratch), None)
    assert st == B.W4_EUNSUPPORTED
    assert "2^32" in B.last_error()


def _swiglu_params(**kw):
    p, _ = _params(**kw)
    if "x_bytes" not in kw:
        p.x_bytes = p.n_tokens * p.top_k * p.k * 4  # gate and up are per routed row
    return p


@pytest.mark.parametrize("kw,status,needle", [
    ({"n_tokens": 1}, B.W4_OK, ""),
    ({"n_tokens": 0}, B.W4_EINVAL, "every size must be positive"),
    ({"n_tokens": 1, "top_k": 0}, B.W4_EINVAL, "top_k=0"),
    ({"n_tokens": 1, "n_experts": 0}, B.W4_EINVAL, "n_experts=0"),
    ({"n_tokens": 1, "k": 2047}, B.W4_EINVAL, "whole number of 32-weight"),
    ({"n_tokens": 1, "expert_stride": 1000}, B.W4_EINVAL, "1000 bytes apart"),
    ({"n_tokens": 1, "x_bytes": 1 * 8 * 2048 * 4 - 1}, B.W4_EINVAL, "gate/up holds 65535 bytes"),
    ({"n_tokens": 1, "w_bytes": 1}, B.W4_EINVAL, "w holds 1 bytes"),
    ({"n_tokens": 1, "ids_bytes": 4}, B.W4_EINVAL, "ids holds 4 bytes"),
    ({"n_tokens": 1, "out_bytes": 4}, B.W4_EINVAL, "out holds 4 bytes"),
    ({"n_tokens": 1, "reserved": 1}, B.W4_EINVAL, "reserved field"),
])
def test_id_swiglu_contract(kw, status, needle):
    p = _swiglu_params(**kw)
    assert B.w4_check_id_swiglu(p) == status
    if status != B.W4_OK:
        assert needle in B.last_error()


@pytest.mark.parametrize("kw", [{"n_tokens": 33, "top_k": 8}, {"n_tokens": 1, "k": 8224}])
def test_id_swiglu_limits_are_reported_before_any_launch(kw):
    import ctypes
    p = _swiglu_params(**kw)
    p.expert_stride = p.n * (p.k // 32) * 18
    p.w_bytes = p.n_experts * p.expert_stride
    assert B.w4_check_id_swiglu(p) == B.W4_OK  # valid: the request is only beyond this library
    st = B.lib().qmm_id_swiglu_q4_0(_fake(), _fake(), _fake(), _fake(), _fake(), ctypes.byref(p), None, None)
    assert st == B.W4_EUNSUPPORTED
    assert "256" in B.last_error() and "8192" in B.last_error()


@pytest.mark.parametrize("args,status", [
    ((4, 4096, 11008, 64, 1), B.W4_OK),
    ((4, 4096, 11008, 64, 0), B.W4_OK),      # both layouts
    ((2, 5, 3, 64, 0), B.W4_OK),             # the page's worked example: blocks straddle rows
    ((0, 5, 3, 2, 1), B.W4_OK),              # empty batch
    ((-1, 5, 3, 2, 1), B.W4_EINVAL),
    ((1, 0, 3, 2, 1), B.W4_EINVAL),
    ((1, 5, 3, 3, 1), B.W4_EINVAL),          # odd block
    ((1, 5, 3, 0, 1), B.W4_EINVAL),
    ((262141, 32, 32, 2, 1), B.W4_EUNSUPPORTED),
])
def test_lut_f32_contract(args, status):
    assert B.w4_check_lut_f32(*args) == status


# ---------------------------------------------------------------- binding shape checks
# The binding checks every tensor's shape against (M, K, N, block) before it touches a device, so a
# wrong shape raises here even with host tensors (no kernel could read or write past a buffer).
import torch


def _affine_host(M=4, K=64, N=32):
    return (torch.zeros((N, K // 8), dtype=torch.int32), torch.zeros((N, K // 32), dtype=torch.bfloat16),
            torch.zeros((N, K // 32), dtype=torch.bfloat16), torch.zeros((M, K), dtype=torch.bfloat16))


@pytest.mark.parametrize("bad", ["w", "scales", "biases", "y"])
def test_binding_rejects_affine_shape_mismatch(bad):
    w, s, b, x = _affine_host()
    y = torch.zeros((4, 32), dtype=torch.bfloat16)
    if bad == "w":
        w = torch.zeros((32, 4), dtype=torch.int32)
    elif bad == "scales":
        s = torch.zeros((32, 1), dtype=torch.bfloat16)
    elif bad == "biases":
        b = torch.zeros((31, 2), dtype=torch.bfloat16)
    else:
        y = torch.zeros((4, 31), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=bad):
        B.qmm_affine4(w, s, b, x, y)


def test_binding_affine_right_shapes_reach_the_device_check():
    w, s, b, x = _affine_host()
    with pytest.raises(TypeError, match="device tensor"):
        B.qmm_affine4(w, s, b, x)


@pytest.mark.parametrize("bad", ["packed", "scales", "y", "book"])
def test_binding_rejects_lut_size_mismatch(bad):
    M, K, N, block = 3, 64, 20, 16
    x = torch.zeros((M, K), dtype=torch.float16)
    packed = torch.zeros(N * K // 2 - (1 if bad == "packed" else 0), dtype=torch.uint8)
    scales = torch.zeros(N * K // block - (1 if bad == "scales" else 0), dtype=torch.float16)
    y = torch.zeros((M, N + (1 if bad == "y" else 0)), dtype=torch.float16)
    book = [0.0] * (15 if bad == "book" else 16)
    with pytest.raises(ValueError, match=bad):
        B.qmm_lut4(x, packed, scales, book, N, block, y=y)
    with pytest.raises(ValueError, match=bad):
        B.qmm_lut4_f32(x.float(), packed, scales.float(), book, N, block, y=None if bad == "y" else y.float()) \
            if bad != "y" else B.qmm_lut4_f32(x.float(), packed, scales.float(), book, N, block, y=y.float())
