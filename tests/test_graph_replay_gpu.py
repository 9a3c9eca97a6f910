"""HIP-graph replays of every entry point reproduce the eager call, bit for bit.

The benchmark times graph replays, so each route is captured here once and replayed several
times, with eager work on the same stream between replays: the output is refilled with NaN
before each replay, so a replay that left any output unwritten, or that depended on state the
eager call left behind (a counter, a scratch list), would show. The kernels' arithmetic is
deterministic (integer atomics only build routing lists, whose order no output depends on),
so the comparison is exact.
"""
import numpy as np
import pytest
import torch

from weight_only_bit_w4_amd import binding as B
from weight_only_bit_w4_amd import synth
from test_parity_gpu import DEV, _affine_dev, _lut_dev, _lut_f32_case, _t

pytestmark = pytest.mark.gpu

REPLAYS = 3
_BITS = {torch.bfloat16: torch.int16, torch.float16: torch.int16, torch.float32: torch.int32}


def _replays_match(call, y, what):
    """call() writes y. The eager result, then REPLAYS replays of one captured call."""
    call()
    torch.cuda.synchronize()
    ref = y.clone()
    assert not torch.isnan(ref.float()).any(), f"{what}: eager output holds NaN"
    side = torch.cuda.Stream()  # a warm-up call on a side stream before capture
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(REPLAYS):
        y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(y.view(_BITS[y.dtype]), ref.view(_BITS[ref.dtype]))
        assert same, f"{what}: replay {i} differs from the eager call"


# (M, K, N): the decode GEMV, the shared-x GEMV form, the weight-tile form with one and two
# x tiles, the register-staged and DMA-ring prefill tiles, and the 64x128 kernel (K % 256 != 0)
AFFINE = [(1, 4096, 512), (3, 512, 256), (32, 1024, 512), (48, 1024, 544), (200, 512, 256), (200, 320, 256),
          (40, 96, 128)]


@pytest.mark.parametrize("M,K,N", AFFINE)
def test_graph_replay_affine(M, K, N):
    print(f"graph replay affine M={M} K={K} N={N}", flush=True)
    c = synth.affine_case(M, K, N, seed=31)
    w, s, b, x = _affine_dev(c)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    fn = B.qmv_affine4 if M == 1 else B.qmm_affine4
    _replays_match(lambda: fn(w, s, b, x, y=y), y, f"affine M={M} K={K} N={N}")


@pytest.mark.parametrize("transpose", [1, 0])
@pytest.mark.parametrize("M,K,N,block", [(130, 512, 256, 64), (3, 512, 200, 32)])
def test_graph_replay_lut4(M, K, N, block, transpose):
    print(f"graph replay lut4 M={M} K={K} N={N} block={block} transpose={transpose}", flush=True)
    c = synth.lut_case(M, K, N, seed=32, block=block)
    x, p, s = _lut_dev(c)
    y = torch.empty((M, N), dtype=torch.float16, device=DEV)
    _replays_match(lambda: B.qmm_lut4(x, p, s, c["book"], N, block, y=y, transpose=transpose), y,
                   f"lut4 M={M} K={K} N={N} block={block} transpose={transpose}")


@pytest.mark.parametrize("transpose", [1, 0])
def test_graph_replay_lut4_f32(transpose):
    M, K, N, block = 4, 512, 300, 64
    print(f"graph replay lut4_f32 transpose={transpose}", flush=True)
    x, packed, scales, book = _lut_f32_case(M, K, N, block, transpose, seed=33)
    xd, pd, sd = _t(x), _t(packed), _t(scales)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    _replays_match(lambda: B.qmm_lut4_f32(xd, pd, sd, book, N, block, y=y, transpose=transpose), y,
                   f"lut4_f32 transpose={transpose}")


# (E, N, K, tokens, top_k): the mat-vec route, the one-launch grouped GEMM, and the two-launch
# form (more than 4096 routed rows: grouping kernel and scratch lists)
MOE = [(8, 96, 256, 4, 2), (8, 96, 256, 60, 4), (16, 64, 256, 600, 8)]


@pytest.mark.parametrize("E,N,K,T,top_k", MOE)
def test_graph_replay_moe(E, N, K, T, top_k):
    print(f"graph replay moe E={E} N={N} K={K} T={T} top_k={top_k}", flush=True)
    c = synth.moe_case(E, N, K, T, top_k, seed=34)
    ids = c["ids"].copy()
    ids[5] = E + 3  # one id naming no expert: its row is written as zeros on every replay
    x, w, idt = _t(c["x"]), _t(c["w"]), _t(ids.view(np.int32))
    scratch = torch.empty(B.qmm_id_q4_0_scratch_bytes(E, T, top_k, K), dtype=torch.uint8, device=DEV)
    out = torch.empty((T * top_k, N), dtype=torch.float32, device=DEV)
    _replays_match(lambda: B.qmm_id_q4_0(x, w, idt, T, top_k, N, K, E, c["expert_stride"], out=out, scratch=scratch),
                   out, f"moe E={E} N={N} K={K} T={T} top_k={top_k}")
    assert int(scratch[:4].view(torch.int32).item()) == 1  # the count of ids naming no expert, not accumulated


def test_graph_replay_moe_swiglu():
    E, N, K, T, top_k = 8, 96, 256, 2, 4
    print("graph replay moe swiglu", flush=True)
    c = synth.moe_swiglu_case(E, N, K, T, top_k, seed=35)
    gate, up, w, idt = _t(c["gate"]), _t(c["up"]), _t(c["w"]), _t(c["ids"].view(np.int32))
    out = torch.empty((T * top_k, N), dtype=torch.float32, device=DEV)
    _replays_match(lambda: B.qmm_id_swiglu_q4_0(gate, up, w, idt, T, top_k, N, K, E, c["expert_stride"], out=out),
                   out, "moe swiglu")
