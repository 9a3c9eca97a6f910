"""The no-allocation expert-routed entry point (qmm_id_q4_0_noalloc) against qmm_id_q4_0 with a caller
scratch buffer: the same kernels, so the outputs must agree with each other and lie within the stated
bound of the oracle; two calls in a row, the second smaller, share the library's fixed scratch. The
size limit is checked on the host before any device work."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from weight_only_bit_w4_amd import binding as B
from weight_only_bit_w4_amd import synth

DEV = "cuda"


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _both(c, ids):
    x, w, idt = _t(c["x"]), _t(c["w"]), _t(ids.view(np.int32))
    args = (c["n_tokens"], c["top_k"], c["N"], c["K"], c["n_experts"], c["expert_stride"])
    bad = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    got = B.qmm_id_q4_0_noalloc(x, w, idt, *args, bad_ids=bad)
    scratch = torch.empty(B.qmm_id_q4_0_scratch_bytes(c["n_experts"], c["n_tokens"], c["top_k"], c["K"]),
                          dtype=torch.uint8, device=DEV)
    ref = B.qmm_id_q4_0(x, w, idt, *args, scratch=scratch)
    torch.cuda.synchronize()
    ref_bad = int(scratch[:4].view(torch.int32).item())
    return got.cpu().numpy().astype(np.float64), ref.cpu().numpy().astype(np.float64), int(bad.item()), ref_bad


@pytest.mark.gpu
def test_no_alloc_matches_caller_scratch_twice_second_smaller():
    # grouped route (more than 32 tokens), then a smaller grouped call, then a mat-vec-route call
    cases = [synth.moe_case(16, 256, 512, 64, 4, seed=41), synth.moe_case(8, 96, 256, 40, 2, seed=42),
             synth.moe_case(8, 64, 128, 3, 2, seed=43)]
    for i, c in enumerate(cases):
        ids = c["ids"].copy()
        ids[5] = c["n_experts"] + 3          # one out-of-range id: a zero row, counted
        got, ref, bad, ref_bad = _both(c, ids)
        assert np.array_equal(got, ref), f"call {i}: no-allocation result differs from the caller-scratch result"
        assert bad == ref_bad == 1, (i, bad, ref_bad)
        acc, _ = oracle.moe_q4_0(c["x"], c["w"], ids, c["n_tokens"], c["top_k"], c["N"], c["K"], c["n_experts"],
                                 c["expert_stride"])
        _, d = oracle.unpack_q4_0(c["w"], c["n_experts"] * c["N"], c["K"])
        tol = oracle.tolerance(acc, c["K"], float(np.abs(c["x"]).max()), float(np.abs(d).max()))
        assert (np.abs(got - acc) <= tol).all(), f"call {i}: outside the stated bound"


def test_no_alloc_rejects_scratch_beyond_its_limit_before_any_device_work():
    # 1024 tokens x K=4096 need 8 MiB of binary16 x in scratch: beyond the fixed 4 MiB
    p = B.IdParams(1024, 8, 1408, 4096, 64, 0, 1408 * 128 * 18, 1024 * 4096 * 4, 64 * 1408 * 128 * 18,
                   1024 * 8 * 4, 1024 * 8 * 1408 * 4)
    fake = ctypes.c_void_p(0x100000)
    st = B.lib().qmm_id_q4_0_noalloc(fake, fake, fake, fake, ctypes.byref(p), None, None)
    assert st == B.W4_EUNSUPPORTED
    assert "4194304" in B.last_error()
