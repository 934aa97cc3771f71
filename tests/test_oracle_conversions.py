"""Pins of the oracle's scalar conversions against library routines (not against itself).

bf16 RNE is checked against torch's float32->bfloat16 conversion; binary16 RNE against
numpy's float32->float16 conversion (then saturated, zero stored as +0); binary16
decode against numpy for all 65,536 patterns.
"""
import numpy as np
import pytest
import torch

import oracle as O


def _torch_bf16_bits(xs: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(xs.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _finite_f32_patterns(rng, n):
    bits = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    return x[np.isfinite(x)]


def test_bf16_rne_against_torch_random_and_ties():
    rng = np.random.default_rng(1)
    xs = list(_finite_f32_patterns(rng, 20000))
    # exact ties and near-ties for every upper half with a finite result
    hi = rng.integers(0, 0x7F7F, size=3000).astype(np.uint32)
    for low in (0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF):
        for s in (0, 0x80000000):
            xs.extend(((hi << 16) | low | s).view(np.float32))
    # subnormal binary32 inputs
    xs.extend(np.array([1, 2, 0x7FFF, 0x8000, 0x18000, 0x7FFFFF], np.uint32).view(np.float32))
    xs = np.array(xs, np.float32)
    xs = xs[np.isfinite(xs)]
    ref = _torch_bf16_bits(xs)
    got = np.array([O.bf16_from_f32(float(v)) for v in xs], np.uint16)
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(hex(xs[i:i+1].view(np.uint32)[0]), hex(ref[i]), hex(got[i])) for i in bad[:5]]


def test_bf16_decode_is_top_half():
    for b in (0x0000, 0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F):
        assert np.float32(O.f32_from_bf16(b)) == np.array([b << 16], np.uint32).view(np.float32)[0]


def _numpy_fp16s_bits(xs: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        h = xs.astype(np.float32).astype(np.float16)
    h = np.where(np.isinf(h), np.sign(h) * np.float16(65504.0), h).astype(np.float16)
    h = np.where(h == 0, np.float16(0.0), h).astype(np.float16)   # +0 for every zero
    return h.view(np.uint16)


def test_fp16s_against_numpy_random_ties_and_range_edges():
    rng = np.random.default_rng(2)
    xs = list(rng.standard_normal(20000).astype(np.float32) * np.float32(3.0))
    xs += list((rng.standard_normal(5000) * 1e-5).astype(np.float32))        # subnormal fp16
    xs += list((rng.standard_normal(5000) * 4e4).astype(np.float32))         # near overflow
    # exact midpoints between consecutive binary16 values (ties), all finite patterns
    allh = np.arange(0, 0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((allh[:-1] + allh[1:]) / 2.0).astype(np.float32)
    xs += list(mids[::7]) + list(-mids[::11])
    xs += [65504.0, 65519.0, 65520.0, 65536.0, 1e9, -1e9, 2.0**30, -(2.0**30),
           0.0, -0.0, 2.0**-25, -(2.0**-25), 2.0**-24, 3 * 2.0**-26, 1e-30]
    xs = np.array(xs, np.float32)
    ref = _numpy_fp16s_bits(xs)
    got = np.array([O.fp16s_from_f32(float(v)) for v in xs], np.uint16)
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(float(xs[i]), hex(ref[i]), hex(got[i])) for i in bad[:5]]


def test_fp16_decode_all_patterns_against_numpy():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    got = np.array([O.f64_from_fp16(int(h)) for h in pats[fin]])
    assert np.array_equal(got, ref[fin])


def test_fp16s_saturates_and_keeps_zero_positive():
    assert O.fp16s_from_f32(1e30) == 0x7BFF
    assert O.fp16s_from_f32(-1e30) == 0xFBFF
    assert O.fp16s_from_f32(-0.0) == 0x0000
    assert O.fp16s_from_f32(-1e-12) == 0x0000          # underflow of a negative value
