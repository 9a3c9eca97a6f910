"""Benchmark of the weight-only 4-bit dequantize-and-multiply hot path on one MI355X.

Headline line: the decode GEMV (affine INT4 group 32, M=1, K=4096, N=14336);
one step = one qmv_affine4 launch (unpack, dequantize, contract, round: every
step of the affine path); value = weight bytes streamed per second. Weight
copies are rotated (>= 512 MiB in total) so the 256 MB Infinity Cache cannot
serve them. The same JSON line carries the other kernels of the path, each
timed over its own back-to-back launches: the tiny affine workload (M=4,
K=N=256, launch-latency bound), the prefill GEMM (M=2048, K=N=4096, TFLOP/s),
the lookup-codebook GEMM (M=512, K=4096, N=11008) and the single-precision
lookup GEMM at 4 rows of x in both weight layouts, and the expert-routed Q4_0
MoE (64 experts, N=1408, K=2048, 128 tokens, top-8; and one decode token,
top-8, on the mat-vec route, plain and with the fused SwiGLU activation), and
qmm_affine4 with 32 rows of x on the decode weights (the small-batch
weight-tile form), each with its roofline fraction against the published peak
and against a measured ceiling (a streaming-read kernel and a matrix-core-only
loop, timed in the same run), plus the CPU oracle: decode GEMVs for a bounded
~10 s sample (the baseline rate) and one full call per workload. --only small
times qmm_affine4 at M = 2..64 on the decode weights.

Each figure is the mean per launch over the timed launches (ms_per_step for
the headline) and the median over the timed graph replays ("us_median").
Launches are captured in HIP graphs (torch.cuda.CUDAGraph over the library's
own launches on the capture stream) and replayed, so the host-side cost of a
call does not pace the GPU; --eager launches them one by one instead (used
under counter collection). Times come from HIP events recorded on the stream
the kernels run on, one between every two replays.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
                       [--only decode|prefill|lut|lut_f32|moe|moe_decode|small|tiny|ceilings] [--eager] [--calib]
"""
from __future__ import annotations

import argparse
import json
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16 matrix cores, TFLOP/s

# HBM bytes per launch (FETCH_SIZE + WRITE_SIZE) from rocprofv3 --pmc runs of
# `bench.py --eager --calib`, each counter scaled by what it reads for a plain
# 256 MiB copy (torch.neg on f32: FETCH_SIZE x 2.0, WRITE_SIZE x 1.0). Each entry
# is tied to the digest of the kernel sources it was measured on and reported
# as null once their code changes (comments and layout aside: see code_digest).
TRAFFIC = {
    "decode": (("w4mi_device.hpp", "affine_gemv.hip"), "7e3a5a299979dcc8", 36831120 + 57347),
    "prefill": (("w4mi_device.hpp", "gemm_w4.hip"), "b5587ba7bc363947", 75864647 + 16803220),
    "lut": (("w4mi_device.hpp", "gemm_w4.hip"), "b5587ba7bc363947", 58303006 + 11816387),
    "lut_kn": (("w4mi_device.hpp", "gemm_w4.hip"), "b5587ba7bc363947", 65502219 + 11785032),
    "small32": (("w4mi_device.hpp", "gemm_w4.hip"), "b5587ba7bc363947", 39082079 + 917504),
    "moe": (("w4mi_device.hpp", "moe_q4_0.hip"), "d873f820bff023d7", 128268590 + 5767200),
    "moe_decode": (("w4mi_device.hpp", "moe_q4_0.hip"), "d873f820bff023d7", 13123794 + 45088),
    "moe_swiglu_decode": (("w4mi_device.hpp", "moe_q4_0.hip"), "d873f820bff023d7", 14108816 + 45056),
    "lut_f32_t1": (("w4mi_device.hpp", "lut_f32.hip"), "2a4765550d6e3759", 26047921 + 176128),
    "lut_f32_t0": (("w4mi_device.hpp", "lut_f32.hip"), "2a4765550d6e3759", 32674713 + 176128),
}


def _code_text(src: str) -> str:
    """C++/HIP source with comments removed and every whitespace run made one space, so a change
    to a comment or to layout leaves it unchanged. String and character literals are kept whole."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def code_digest(paths) -> str:
    """First 16 hex of the sha256 over the comment-free code of `paths`, in order."""
    import hashlib

    h = hashlib.sha256()
    for path in paths:
        with open(path, encoding="utf-8") as f:
            h.update(_code_text(f.read()).encode())
    return h.hexdigest()[:16]


def traffic(name: str):
    """Measured HBM bytes per launch of `name`, or None if its sources' code changed since."""
    import os

    if name not in TRAFFIC:
        return None
    sources, digest, nbytes = TRAFFIC[name]
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "weight_only_bit_w4_amd", "csrc")
    return nbytes if code_digest([os.path.join(csrc, s) for s in sources]) == digest else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default=None, choices=["decode", "prefill", "lut", "lut_f32", "moe", "moe_decode", "small",
                                                    "tiny", "ceilings"],
                    help="time one kernel only")
    ap.add_argument("--eager", action="store_true", help="launch one by one instead of replaying graphs")
    ap.add_argument("--calib", action="store_true",
                    help="also run a plain 256 MiB copy kernel (counter calibration)")
    return ap.parse_args()


def oracle_free_f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns to f32 (numpy's own conversion)."""
    return np.ascontiguousarray(bits).view(np.float16).astype(np.float32)


def rotation(bytes_per_copy: int, min_total: int = 512 * 2**20) -> int:
    return max(2, -(-min_total // bytes_per_copy))


class Timer:
    """Times `steps` launches of launch(i) with HIP events on torch's current
    stream (the stream the binding enqueues on), after `warmup` launches."""

    def __init__(self, torch, eager: bool):
        self.torch = torch
        self.eager = eager

    def _graph(self, launch, first: int, count: int):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(first, first + count):
                launch(i)
        return g

    def run(self, launch, steps: int, warmup: int, chunk: int = 60) -> float:
        """Mean ms per launch over `steps` launches (see run_stats)."""
        return self.run_stats(launch, steps, warmup, chunk)[0]

    def run_stats(self, launch, steps: int, warmup: int, chunk: int = 60):
        """(mean ms per launch, median ms per launch) over `steps` launches: the launches run as
        back-to-back replays of a graph of `chunk` launches, each replay between two events on the
        launch stream; the median is taken over the replays' per-launch times (eager mode: one
        launch per event pair)."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        if self.eager:
            for i in range(warmup):
                launch(i)
            chunk = 1
            plan = None
        else:
            # Eager warm-up on a side stream (default priority), then capture.
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for i in range(3):
                    launch(i)
            stream.wait_stream(side)
            torch.cuda.synchronize()
            chunk = max(1, min(chunk, steps))
            full = self._graph(launch, 0, chunk)
            rest = self._graph(launch, 0, steps % chunk) if steps % chunk else None
            plan = [(full, chunk)] * (steps // chunk) + ([(rest, steps % chunk)] if rest is not None else [])
            # Warm-up: the requested launches, and at least ~0.2 s of
            # back-to-back work so the clocks have settled before timing.
            torch.cuda.synchronize()
            t_end = time.perf_counter() + 0.2
            n = 0
            while n < max(1, warmup // chunk) or time.perf_counter() < t_end:
                full.replay()
                n += 1
                if n % 8 == 0:
                    torch.cuda.synchronize()
        torch.cuda.synchronize()
        count = steps if plan is None else len(plan)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(count + 1)]
        marks[0].record(stream)
        for r in range(count):
            if plan is None:
                launch(r)
            else:
                plan[r][0].replay()
            marks[r + 1].record(stream)
        torch.cuda.synchronize()
        sizes = [1] * count if plan is None else [n for _, n in plan]
        per = [marks[r].elapsed_time(marks[r + 1]) / sizes[r] for r in range(count)]
        total = marks[0].elapsed_time(marks[count])
        return total / steps, float(np.median(per))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the path runs on one GPU (got --gpus {args.gpus}); "
              "sharding across GPUs is a design note, not part of this benchmark", file=sys.stderr)
        sys.exit(2)
    import torch

    from weight_only_bit_w4_amd import binding as B
    from weight_only_bit_w4_amd import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    B.lib()  # fail loudly before anything else if the library is missing
    dev = "cuda"
    timer = Timer(torch, args.eager)
    steps, warmup = args.steps, args.warmup

    def to_dev(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(dtype) if dtype is not None else t).to(dev)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    result = {}

    if args.calib:
        a = torch.ones(64 * 2**20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        log("calibration copy: torch.neg over 256 MiB f32 (reads 268435456 B, writes 268435456 B), 5 launches")
        del a, b

    # ------------------------------------------------------------ decode GEMV (headline)
    c2 = synth.decode_affine()
    M, K, N = c2["M"], c2["K"], c2["N"]
    wbytes2 = N * K // 2 + 2 * (N * K // 32) * 2
    if args.only in (None, "decode"):
        ncopy = rotation(wbytes2)
        ws = [to_dev(c2["w"].view(np.int32))]
        ss = [to_dev(c2["scales"].view(np.int16), torch.bfloat16)]
        bs = [to_dev(c2["biases"].view(np.int16), torch.bfloat16)]
        for _ in range(ncopy - 1):
            ws.append(ws[0].clone())
            ss.append(ss[0].clone())
            bs.append(bs[0].clone())
        x2 = to_dev(c2["x"].view(np.int16), torch.bfloat16)
        y2 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def decode_step(i):
            j = i % ncopy
            B.qmv_affine4(ws[j], ss[j], bs[j], x2, y2)

        log(f"decode: qmv_affine4 M=1 K={K} N={N}, {ncopy} weight copies, {steps} launches")
        ms, med = timer.run_stats(decode_step, steps, warmup, chunk=ncopy * 4)
        result["decode"] = {"ms": ms, "ms_median": med, "GBps": wbytes2 / (ms * 1e-3) / 1e9, "copies": ncopy}
        del ws, ss, bs, x2, y2

    # ------------------------------------------------------------ prefill GEMM
    if args.only in (None, "prefill"):
        c3 = synth.prefill_affine()
        M3, K3, N3 = c3["M"], c3["K"], c3["N"]
        w3 = to_dev(c3["w"].view(np.int32))
        s3 = to_dev(c3["scales"].view(np.int16), torch.bfloat16)
        b3 = to_dev(c3["biases"].view(np.int16), torch.bfloat16)
        x3 = to_dev(c3["x"].view(np.int16), torch.bfloat16)
        y3 = torch.empty((M3, N3), dtype=torch.bfloat16, device=dev)
        n3 = max(20, steps // 10)
        log(f"prefill: qmm_affine4 M={M3} K={K3} N={N3}, {n3} launches")
        ms, med = timer.run_stats(lambda i: B.qmm_affine4(w3, s3, b3, x3, y3), n3, max(5, warmup // 5), chunk=10)
        flops = 2.0 * M3 * N3 * K3
        result["prefill"] = {"ms": ms, "ms_median": med, "TFLOPs": flops / (ms * 1e-3) / 1e12, "launches": n3}
        del w3, s3, b3, x3, y3

    # ------------------------------------------------------------ lookup-codebook GEMM
    if args.only in (None, "lut"):
        c4 = synth.lut_matmul_case()
        M4, K4, N4, blk = c4["M"], c4["K"], c4["N"], c4["block"]
        x4 = to_dev(c4["x"].view(np.int16), torch.float16)
        p4 = to_dev(c4["packed"])
        s4 = to_dev(c4["scales"].view(np.int16), torch.float16)
        y4 = torch.empty((M4, N4), dtype=torch.float16, device=dev)
        n4 = max(20, steps // 10)
        log(f"lut: qmm_lut4 M={M4} K={K4} N={N4} block {blk}, {n4} launches")
        ms, med = timer.run_stats(lambda i: B.qmm_lut4(x4, p4, s4, c4["book"], N4, blk, y=y4), n4,
                                  max(5, warmup // 5), chunk=10)
        flops = 2.0 * M4 * N4 * K4
        result["lut"] = {"ms": ms, "ms_median": med, "TFLOPs": flops / (ms * 1e-3) / 1e12, "launches": n4}
        # the same bytes read as a weight stored [K, N] (transpose == 0): the matrix-core [K, N] route
        log(f"lut [K, N]: qmm_lut4 transpose=0 M={M4} K={K4} N={N4} block {blk}, {n4} launches")
        ms, med = timer.run_stats(lambda i: B.qmm_lut4(x4, p4, s4, c4["book"], N4, blk, y=y4, transpose=0), n4,
                                  max(5, warmup // 5), chunk=10)
        result["lut_kn"] = {"ms": ms, "ms_median": med, "TFLOPs": flops / (ms * 1e-3) / 1e12, "launches": n4}
        del x4, p4, s4, y4

    # ------------------------------------------------------------ lookup codebook, single precision, 4 rows
    if args.only in (None, "lut_f32"):
        c8 = synth.lut_matmul_case()
        K8, N8, blk8, M8 = c8["K"], c8["N"], c8["block"], 4
        p8 = [to_dev(c8["packed"])]
        s8 = [to_dev(oracle_free_f16_to_f32(c8["scales"]))]
        wbytes8 = p8[0].numel() + s8[0].numel() * 4
        ncopy8 = rotation(wbytes8)
        for _ in range(ncopy8 - 1):
            p8.append(p8[0].clone())
            s8.append(s8[0].clone())
        x8 = to_dev(np.random.default_rng(8).standard_normal((M8, K8)).astype(np.float32))
        y8 = torch.empty((M8, N8), dtype=torch.float32, device=dev)
        n8 = max(200, steps // 4)
        for t8 in (1, 0):
            log(f"lut f32: qmm_lut4_f32 M={M8} K={K8} N={N8} block {blk8} transpose={t8}, {ncopy8} weight copies, "
                f"{n8} launches")
            ms, med = timer.run_stats(lambda i: B.qmm_lut4_f32(x8, p8[i % ncopy8], s8[i % ncopy8], c8["book"], N8, blk8,
                                                               y=y8, transpose=t8), n8, max(10, warmup // 2),
                                      chunk=ncopy8 * 2)
            result[f"lut_f32_t{t8}"] = {"ms": ms, "ms_median": med, "GBps": wbytes8 / (ms * 1e-3) / 1e9, "M": M8}
        del p8, s8, x8, y8

    # ------------------------------------------------------------ expert-routed Q4_0
    if args.only in (None, "moe"):
        c5 = synth.moe_q4_0_case()
        E, N5, K5, T, top_k = c5["n_experts"], c5["N"], c5["K"], c5["n_tokens"], c5["top_k"]
        wbytes5 = c5["w"].size
        ncopy5 = rotation(wbytes5)
        w5 = [to_dev(c5["w"])]
        for _ in range(ncopy5 - 1):
            w5.append(w5[0].clone())
        x5 = to_dev(c5["x"])
        ids5 = to_dev(c5["ids"].view(np.int32))
        out5 = torch.empty((T * top_k, N5), dtype=torch.float32, device=dev)
        scratch5 = torch.empty(B.qmm_id_q4_0_scratch_bytes(E, T, top_k, K5), dtype=torch.uint8, device=dev)
        n5 = max(60, steps // 4)
        log(f"moe: qmm_id_q4_0 E={E} N={N5} K={K5} tokens={T} top_k={top_k}, {ncopy5} weight copies, {n5} launches")
        ms, med = timer.run_stats(lambda i: B.qmm_id_q4_0(x5, w5[i % ncopy5], ids5, T, top_k, N5, K5, E,
                                                          c5["expert_stride"], out=out5, scratch=scratch5),
                                  n5, max(5, warmup // 2), chunk=ncopy5 * 2)
        result["moe"] = {"ms": ms, "ms_median": med, "GBps": wbytes5 / (ms * 1e-3) / 1e9, "copies": ncopy5,
                         "launches": n5}
        del w5, x5, ids5, out5, scratch5

    # ------------------------------------------------------------ expert-routed Q4_0, one decode token
    if args.only in (None, "moe_decode"):
        c6 = synth.moe_q4_0_case()
        E, N6, K6, top_k6 = c6["n_experts"], c6["N"], c6["K"], c6["top_k"]
        expert_bytes = N6 * (K6 // 32) * 18
        wbytes6 = top_k6 * expert_bytes  # the selected experts' weights, read once
        # Rotate over disjoint expert sets (a seeded permutation of all experts,
        # top_k at a time) and weight copies, so that successive calls touch
        # >= 512 MiB before any byte comes round again.
        perm = np.random.default_rng(6).permutation(E).astype(np.uint32)
        sets = [to_dev(perm[i:i + top_k6].view(np.int32)) for i in range(0, E - top_k6 + 1, top_k6)]
        ncopy6 = rotation(wbytes6 * len(sets))
        w6 = [to_dev(c6["w"])]
        for _ in range(ncopy6 - 1):
            w6.append(w6[0].clone())
        x6 = to_dev(c6["x"][:1])
        out6 = torch.empty((top_k6, N6), dtype=torch.float32, device=dev)
        scratch6 = torch.empty(B.qmm_id_q4_0_scratch_bytes(E, 1, top_k6, K6), dtype=torch.uint8, device=dev)
        n6 = max(200, steps // 2)
        combos = ncopy6 * len(sets)
        log(f"moe decode: qmm_id_q4_0 E={E} N={N6} K={K6} tokens=1 top_k={top_k6}, {len(sets)} expert sets x "
            f"{ncopy6} weight copies, {n6} launches")
        ms, med = timer.run_stats(lambda i: B.qmm_id_q4_0(x6, w6[(i // len(sets)) % ncopy6], sets[i % len(sets)], 1,
                                                          top_k6, N6, K6, E, c6["expert_stride"], out=out6,
                                                          scratch=scratch6),
                                  n6, max(10, warmup), chunk=combos * 2)
        result["moe_decode"] = {"ms": ms, "ms_median": med, "GBps": wbytes6 / (ms * 1e-3) / 1e9, "copies": ncopy6,
                                "sets": len(sets), "launches": n6}
        # The fused SwiGLU form on the same experts: gate and up per routed row.
        c7 = synth.moe_swiglu_decode_case()
        g7, u7 = to_dev(c7["gate"]), to_dev(c7["up"])
        log(f"moe swiglu decode: qmm_id_swiglu_q4_0 E={E} N={N6} K={K6} tokens=1 top_k={top_k6}, same rotation, "
            f"{n6} launches")
        ms, med = timer.run_stats(lambda i: B.qmm_id_swiglu_q4_0(g7, u7, w6[(i // len(sets)) % ncopy6],
                                                                 sets[i % len(sets)], 1, top_k6, N6, K6, E,
                                                                 c6["expert_stride"], out=out6),
                                  n6, max(10, warmup), chunk=combos * 2)
        result["moe_swiglu_decode"] = {"ms": ms, "ms_median": med, "GBps": wbytes6 / (ms * 1e-3) / 1e9, "launches": n6}
        del w6, x6, sets, out6, scratch6, g7, u7

    # ------------------------------------------------------------ small batch (32 rows of x)
    if args.only is None:
        # qmm_affine4 with 32 rows of x on the decode weights: the weight-tile form.
        ncopy = rotation(wbytes2)
        ws = [to_dev(c2["w"].view(np.int32))]
        ss = [to_dev(c2["scales"].view(np.int16), torch.bfloat16)]
        bs = [to_dev(c2["biases"].view(np.int16), torch.bfloat16)]
        for _ in range(ncopy - 1):
            ws.append(ws[0].clone())
            ss.append(ss[0].clone())
            bs.append(bs[0].clone())
        xs = to_dev(np.random.default_rng(7).standard_normal((32, K)).astype(np.float32)).to(torch.bfloat16)
        ys = torch.empty((32, N), dtype=torch.bfloat16, device=dev)
        log(f"small batch: qmm_affine4 M=32 K={K} N={N}, {ncopy} weight copies, 600 launches")
        ms, med = timer.run_stats(lambda i: B.qmm_affine4(ws[i % ncopy], ss[i % ncopy], bs[i % ncopy], xs, ys), 600, 30,
                                  chunk=ncopy * 4)
        result["small32"] = {"ms": ms, "ms_median": med, "GBps": wbytes2 / (ms * 1e-3) / 1e9}
        del ws, ss, bs, xs, ys

    # ------------------------------------------------------------ tiny affine workload (launch-latency bound)
    if args.only in (None, "tiny"):
        c1 = synth.tiny_affine()
        M1, K1, N1 = c1["M"], c1["K"], c1["N"]
        w1 = to_dev(c1["w"].view(np.int32))
        s1 = to_dev(c1["scales"].view(np.int16), torch.bfloat16)
        b1 = to_dev(c1["biases"].view(np.int16), torch.bfloat16)
        x1 = to_dev(c1["x"].view(np.int16), torch.bfloat16)
        y1 = torch.empty((M1, N1), dtype=torch.bfloat16, device=dev)
        log(f"tiny: qmm_affine4 M={M1} K={K1} N={N1}, 2000 launches")
        ms, med = timer.run_stats(lambda i: B.qmm_affine4(w1, s1, b1, x1, y1), 2000, 50, chunk=100)
        result["tiny"] = {"ms": ms, "ms_median": med, "M": M1, "K": K1, "N": N1}
        del w1, s1, b1, x1, y1

    # ------------------------------------------------------------ measured ceilings
    if args.only in (None, "ceilings"):
        sink = torch.zeros(1024, dtype=torch.int32, device=dev)
        big = torch.empty(512 * 2**20 // 4, dtype=torch.int32, device=dev).fill_(1)
        log("ceiling: streaming read of 512 MiB, 40 launches")
        ms, med = timer.run_stats(lambda i: B.w4_ceiling_stream_read(big, sink), 40, 5, chunk=4)
        read_big = big.numel() * 4 / (ms * 1e-3) / 1e9
        # the decode weights' footprint (36.7 MB), rotated over 512 MiB as the decode GEMV is
        nview = big.numel() * 4 // wbytes2
        views = [big[j * (wbytes2 // 4):(j + 1) * (wbytes2 // 4)] for j in range(nview)]
        log(f"ceiling: streaming read of {wbytes2} B, {nview} rotated views, 1000 launches")
        ms2, med2 = timer.run_stats(lambda i: B.w4_ceiling_stream_read(views[i % nview], sink), 1000, 50,
                                    chunk=nview * 4)
        # The vendor library's plain half-precision GEMM of the prefill and lookup shapes (no
        # dequantization): what a tuned GEMM reaches on these shapes on this GPU.
        lib_gemm = {}
        for tag, (Mg, Kg, Ng) in (("prefill shape", (2048, 4096, 4096)), ("lookup shape", (512, 4096, 11008))):
            ga = torch.randn((Mg, Kg), device=dev).to(torch.float16)
            gb = torch.randn((Kg, Ng), device=dev).to(torch.float16)   # [K, N] contiguous
            gc = torch.empty((Mg, Ng), dtype=torch.float16, device=dev)
            log(f"ceiling: torch.matmul fp16 {Mg}x{Kg}x{Ng} (hipBLASLt), 100 launches")
            msg, medg = timer.run_stats(lambda i: torch.matmul(ga, gb, out=gc), 100, 10, chunk=10)
            lib_gemm[tag] = {"M": Mg, "K": Kg, "N": Ng, "us": round(msg * 1e3, 2),
                             "TFLOPs": round(2.0 * Mg * Kg * Ng / (msg * 1e-3) / 1e12, 1)}
            del ga, gb, gc
        iters = 4096
        log(f"ceiling: f16 matrix-core loop, {iters} x 4 MFMA per wavefront, 20 launches")
        ms3, med3 = timer.run_stats(lambda i: B.w4_ceiling_mfma(sink, iters), 20, 3, chunk=2)
        mfma_flop = 2 * 256 * 4 * 4 * iters * 32768
        result["ceilings"] = {
            "hbm_stream_read": {"GBps": round(read_big, 1), "bytes": big.numel() * 4, "ms": round(ms, 5)},
            "hbm_stream_read_decode_footprint": {"GBps": round(wbytes2 / (ms2 * 1e-3) / 1e9, 1), "bytes": wbytes2,
                                                 "us": round(ms2 * 1e3, 3), "us_median": round(med2 * 1e3, 3)},
            "mfma_f16": {"TFLOPs": round(mfma_flop / (ms3 * 1e-3) / 1e12, 1), "ms": round(ms3, 4)},
            "library_fp16_gemm": lib_gemm,
        }
        del big, views, sink

    # ------------------------------------------------------------ small batches (on request only)
    if args.only == "small":
        # qmm_affine4 with a few rows of x on the decode weights (not part of the default line).
        ncopy = rotation(wbytes2)
        ws = [to_dev(c2["w"].view(np.int32))]
        ss = [to_dev(c2["scales"].view(np.int16), torch.bfloat16)]
        bs = [to_dev(c2["biases"].view(np.int16), torch.bfloat16)]
        for _ in range(ncopy - 1):
            ws.append(ws[0].clone())
            ss.append(ss[0].clone())
            bs.append(bs[0].clone())
        rng = np.random.default_rng(7)
        small = {}
        for Ms in (2, 4, 8, 16, 32, 64):
            xs = to_dev(rng.standard_normal((Ms, K)).astype(np.float32)).to(torch.bfloat16)
            ys = torch.empty((Ms, N), dtype=torch.bfloat16, device=dev)
            ms = timer.run(lambda i: B.qmm_affine4(ws[i % ncopy], ss[i % ncopy], bs[i % ncopy], xs, ys), 600, 30,
                           chunk=ncopy * 4)
            small[f"M={Ms}"] = {"ms": round(ms, 5), "GBps": round(wbytes2 / (ms * 1e-3) / 1e9, 1)}
            log(f"small batch: qmm_affine4 M={Ms} K={K} N={N}: {ms * 1e3:.2f} us")
        result["small"] = small
        del ws, ss, bs

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu and args.only in (None, "decode"):
        import oracle
        c = c2
        log("cpu baseline: oracle decode GEMVs on the host cores (about 10 s)")
        oracle.affine(c["w"], c["scales"], c["biases"], c["x"], 1, K, N)  # warm (build, page-in)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.affine(c["w"], c["scales"], c["biases"], c["x"], 1, K, N)
            reps += 1
            el = time.perf_counter() - t0
            if el > 10.0 or reps >= 400:
                break
        cpu = {"value": round(wbytes2 * reps / el / 1e9, 4), "unit": "GB/s", "cores": oracle.threads(),
               "kind": "oracle",
               "sample": f"{reps} full decode GEMVs (M=1, K={K}, N={N}) in {el:.1f} s, weight bytes per second"}

        # One full oracle call per workload (dequantize, fp64 accumulate, round): the small ones after a
        # warm-up as the median of 3 calls, the prefill and lookup GEMMs (seconds each) once.
        def timed(fn, runs):
            if runs > 1:
                fn()
            ts = []
            for _ in range(runs):
                t = time.perf_counter()
                fn()
                ts.append(time.perf_counter() - t)
            return round(float(np.median(ts)) * 1e3, 3), runs

        c1 = synth.tiny_affine()
        c3 = synth.prefill_affine()
        c4 = synth.lut_matmul_case()
        c5 = synth.moe_q4_0_case()
        log("cpu baseline: one oracle call per workload (prefill and lookup GEMMs run once, about 15 s)")
        table = {}
        for name, fn, runs in (
                ("tiny affine M=4 K=256 N=256",
                 lambda: oracle.affine(c1["w"], c1["scales"], c1["biases"], c1["x"], c1["M"], c1["K"], c1["N"]), 3),
                ("decode GEMV M=1 K=4096 N=14336",
                 lambda: oracle.affine(c2["w"], c2["scales"], c2["biases"], c2["x"], 1, K, N), 3),
                ("prefill GEMM M=2048 K=4096 N=4096",
                 lambda: oracle.affine(c3["w"], c3["scales"], c3["biases"], c3["x"], c3["M"], c3["K"], c3["N"]), 1),
                ("lookup GEMM M=512 K=4096 N=11008",
                 lambda: oracle.lut4(c4["x"], c4["packed"], c4["scales"], c4["book"], c4["M"], c4["K"], c4["N"],
                                     c4["block"]), 1),
                ("MoE Q4_0 E=64 N=1408 K=2048 tokens=128 top-8",
                 lambda: oracle.moe_q4_0(c5["x"], c5["w"], c5["ids"], c5["n_tokens"], c5["top_k"], c5["N"], c5["K"],
                                         c5["n_experts"], c5["expert_stride"]), 3)):
            ms_cpu, n = timed(fn, runs)
            table[name] = {"ms": ms_cpu, "calls": n}
            log(f"cpu baseline: {name}: {ms_cpu:.1f} ms")
        cpu["oracle_ms"] = table

    # ------------------------------------------------------------ report
    mode = "eager launches" if args.eager else "HIP-graph replays of back-to-back launches"
    out = {
        "metric": "W4 qmm TFLOP/s (prefill) + weight GB/s (decode GEMV), % of MI355X roofline",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy draws with the workloads' shapes and distributions)",
        "timing": mode,
    }

    if "decode" in result:
        d = result["decode"]
        out.update({
            "value": round(d["GBps"], 2),
            "unit": "GB/s",
            "ms_per_step": round(d["ms"], 6),
            "us_median_per_step": round(d["ms_median"] * 1e3, 3),
            "config": {"workload": "decode GEMV, affine INT4 group 32: x bf16 [1, 4096] . W[14336, 4096]^T",
                       "M": 1, "K": K, "N": N, "group_size": 32, "weight_bytes": wbytes2,
                       "weight_copies_rotated": d["copies"]},
            "roofline": {"bound": "hbm", "achieved": round(d["GBps"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(d["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic("decode")},
        })
        if "ceilings" in result:
            ceil = result["ceilings"]["hbm_stream_read_decode_footprint"]["GBps"]
            out["roofline"]["measured_ceiling"] = ceil
            out["roofline"]["frac_of_measured_ceiling"] = round(d["GBps"] / ceil, 4)
    comps = {}
    if "prefill" in result:
        p = result["prefill"]
        comps["prefill_gemm"] = {
            "workload": "qmm_affine4 M=2048 K=4096 N=4096", "ms": round(p["ms"], 5),
            "value": round(p["TFLOPs"], 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(p["TFLOPs"], 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(p["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic("prefill")}}
    if "lut" in result:
        p = result["lut"]
        comps["lut_gemm"] = {
            "workload": "qmm_lut4 M=512 K=4096 N=11008 block 64", "ms": round(p["ms"], 5),
            "value": round(p["TFLOPs"], 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(p["TFLOPs"], 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(p["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic("lut")}}
    if "lut_kn" in result:
        p = result["lut_kn"]
        comps["lut_gemm_kn"] = {
            "workload": "qmm_lut4 M=512 K=4096 N=11008 block 64, W stored [K, N] (transpose=0)", "ms": round(p["ms"], 5),
            "value": round(p["TFLOPs"], 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(p["TFLOPs"], 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(p["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic("lut_kn")}}
    if "moe" in result:
        p = result["moe"]
        comps["moe_q4_0"] = {
            "workload": "qmm_id_q4_0 E=64 N=1408 K=2048 tokens=128 top_k=8 (one-launch grouped GEMM)",
            "ms": round(p["ms"], 5), "value": round(p["GBps"], 2), "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(p["GBps"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(p["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic("moe")}}
    if "moe_decode" in result:
        p = result["moe_decode"]
        comps["moe_q4_0_decode"] = {
            "workload": "qmm_id_q4_0 E=64 N=1408 K=2048 tokens=1 top_k=8 (mat-vec route; 8 experts' weights)",
            "ms": round(p["ms"], 5), "value": round(p["GBps"], 2), "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(p["GBps"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(p["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic("moe_decode")}}
    if "moe_swiglu_decode" in result:
        p = result["moe_swiglu_decode"]
        comps["moe_swiglu_q4_0_decode"] = {
            "workload": "qmm_id_swiglu_q4_0 E=64 N=1408 K=2048 tokens=1 top_k=8 (fused silu(gate)*up; 8 experts' weights)",
            "ms": round(p["ms"], 5), "value": round(p["GBps"], 2), "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(p["GBps"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(p["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic("moe_swiglu_decode")}}
    for t8, layout in ((1, "[N, K]"), (0, "[K, N]")):
        if f"lut_f32_t{t8}" in result:
            p = result[f"lut_f32_t{t8}"]
            comps[f"lut_f32_transpose{t8}"] = {
                "workload": f"qmm_lut4_f32 M=4 K=4096 N=11008 block 64, W {layout}, f32 x/scales/y",
                "ms": round(p["ms"], 5), "value": round(p["GBps"], 2), "unit": "GB/s",
                "roofline": {"bound": "hbm", "achieved": round(p["GBps"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(p["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic(f"lut_f32_t{t8}")}}
    if "small32" in result:
        p = result["small32"]
        comps["small_batch_gemm"] = {
            "workload": f"qmm_affine4 M=32 K={K} N={N} (decode weights, weight-tile form)",
            "ms": round(p["ms"], 5), "value": round(p["GBps"], 2), "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(p["GBps"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(p["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic("small32")}}
    if "small" in result:
        comps["affine_small_batch"] = {"workload": f"qmm_affine4 M=2..64 K={K} N={N} (decode weights)",
                                       "unit": "GB/s weights", "points": result["small"]}
    if "tiny" in result:
        p = result["tiny"]
        comps["tiny_affine"] = {"workload": "qmm_affine4 M=4 K=256 N=256 (launch-latency bound)",
                                "us": round(p["ms"] * 1e3, 3), "us_median": round(p["ms_median"] * 1e3, 3)}
    for name, key in (("prefill_gemm", "prefill"), ("lut_gemm", "lut"), ("lut_gemm_kn", "lut_kn"), ("moe_q4_0", "moe"),
                      ("moe_q4_0_decode", "moe_decode"), ("moe_swiglu_q4_0_decode", "moe_swiglu_decode"),
                      ("lut_f32_transpose1", "lut_f32_t1"), ("lut_f32_transpose0", "lut_f32_t0"),
                      ("small_batch_gemm", "small32")):
        if name in comps and key in result:
            comps[name]["us_median"] = round(result[key]["ms_median"] * 1e3, 3)
            if "ceilings" in result:
                r = comps[name]["roofline"]
                ceil = (result["ceilings"]["mfma_f16"]["TFLOPs"] if r["bound"] == "mfma"
                        else result["ceilings"]["hbm_stream_read"]["GBps"])
                r["measured_ceiling"] = ceil
                r["frac_of_measured_ceiling"] = round(r["achieved"] / ceil, 4)
    if comps:
        out["components"] = comps
    if "ceilings" in result:
        out["ceilings"] = result["ceilings"]
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
