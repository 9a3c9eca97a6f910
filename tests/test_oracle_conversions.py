"""Pins of the oracle's own bf16 / fp16 conversions against numpy and torch.

The oracle writes its 16-bit float conversions from the IEEE-754 binary16 and
bfloat16 definitions (round to nearest, ties to even). Here they are checked
exhaustively over every 16-bit pattern and, for the narrowing direction, over
all representable values, every midpoint between neighbours (the ties) and a
large random sample of binary32 bit patterns.
"""
import numpy as np
import torch

import oracle


def _same_bits_or_both_nan(a_bits, b_bits, nan_mask):
    ok = (a_bits == b_bits) | nan_mask
    return bool(ok.all())


def test_f16_to_f32_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_to_f32_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f16_narrowing_probe():
    rng = np.random.default_rng(1)
    finite16 = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite16 = finite16[np.isfinite(finite16)].astype(np.float64)
    vals = np.sort(np.unique(finite16))
    mids = (vals[:-1] + vals[1:]) / 2.0                     # exact ties
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                           np.nextafter(mids.astype(np.float32), np.float32(-np.inf))])
    rnd = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
    edge = np.array([65504, 65519.99, 65520, 65535, 1e6, 5.96e-8, 2.98e-8, 2.99e-8, 1e-9, 0.0, -0.0,
                     np.inf, -np.inf], np.float32)
    return np.concatenate([vals.astype(np.float32), mids.astype(np.float32), near, rnd, edge])


def test_f32_to_f16_round_nearest_even():
    f = _f16_narrowing_probe()
    ours = oracle.f32_to_f16(f)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    nan = np.isnan(f)
    assert _same_bits_or_both_nan(ours, ref, nan)
    assert np.all((ours[nan] & 0x7C00) == 0x7C00) and np.all((ours[nan] & 0x03FF) != 0)


def test_f32_to_bf16_round_nearest_even():
    rng = np.random.default_rng(2)
    rnd = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # exact ties: low 16 bits == 0x8000 with both parities of the kept part
    ties = (rng.integers(0, 2**16, size=4096, dtype=np.uint32) << 16) | 0x8000
    bits = np.concatenate([rnd, ties, np.array([0x7F7FFFFF, 0x7F7F8000, 0xFF7F8000, 0x00008000, 0x00018000],
                                               np.uint32)])
    f = bits.view(np.float32)
    ours = oracle.f32_to_bf16(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert _same_bits_or_both_nan(ours, ref, nan)


def test_round_trip_is_identity_on_representable_values():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.f16_to_f32(h)
    fin = np.isfinite(f)
    assert np.array_equal(oracle.f32_to_f16(f[fin]), h[fin])
    b = oracle.bf16_to_f32(h)
    fin = np.isfinite(b) | np.isinf(b)
    assert np.array_equal(oracle.f32_to_bf16(b[fin]), h[fin])
