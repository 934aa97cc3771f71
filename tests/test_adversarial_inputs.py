"""The crafted inputs of the edge-case GPU tests reach the branches they are meant for (CPU
only; the oracle classifies each block): for every code width, some block's symmetric
scale is binary16 zero from a nonzero block, a binary16 subnormal, saturated at +-65504,
and some element lands exactly on a rounding tie of x / d; the affine encoder sees a zero
step (constant block), a saturated minimum and a tie; and the KVarN pages include the
channel-guard page."""
import numpy as np
import pytest

import oracle as O

import adversarial_inputs as A


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("N", (2, 3, 4, 5, 6, 8))
def test_catalog_reaches_symmetric_branches(N):
    seen = set()
    for b in A.block_catalog(N):
        x = b.astype(np.float32)
        d, u = O.encode_block_q0(N, x)
        mag = d & 0x7FFF
        if d == 0 and np.any(x != 0):
            seen.add("zero_scale_nonzero_block")
        if d == 0 and np.all(x == 0):
            seen.add("all_zero")
        if 0 < mag < 0x0400:
            seen.add("subnormal_scale")
        if mag == 0x7BFF:
            seen.add("saturated_scale")
        if mag and mag < 0x7C00:
            df = O.f64_from_fp16(d)
            t = x.astype(np.float64) / df
            if np.any(np.abs(t - np.floor(t)) == 0.5):
                seen.add("rounding_tie")
        mx, mn = x.max(), x.min()
        if mx == -mn and mx != 0:
            seen.add("tied_extremes")
    want = {"zero_scale_nonzero_block", "all_zero", "subnormal_scale", "saturated_scale",
            "rounding_tie", "tied_extremes"}
    assert want <= seen, want - seen


@pytest.mark.parametrize("N", (2, 3, 4, 5, 6, 8))
def test_catalog_reaches_affine_branches(N):
    seen = set()
    for b in A.block_catalog(N):
        x = b.astype(np.float32)
        d, m, u = O.encode_block_q1(N, x)
        if d == 0:
            seen.add("zero_step")
        if (m & 0x7FFF) == 0x7BFF:
            seen.add("saturated_minimum")
        if d and (d & 0x7FFF) < 0x7C00:
            t = (x.astype(np.float64) - O.f64_from_fp16(m)) / O.f64_from_fp16(d)
            if np.any(np.abs(t - np.floor(t)) == 0.5):
                seen.add("rounding_tie")
    assert {"zero_step", "saturated_minimum", "rounding_tie"} <= seen, seen


def test_pages_include_channel_guard():
    pages = A.crafted_pages()
    hit = 0
    for X in pages:
        _, _, cs = O.encode_page_kvarn(4, X)
        Y = np.array([O.fwht128(r) for r in _f32(X)])
        if np.any(cs == 0x3C00) and np.any(Y != 0):
            hit += 1
    assert hit >= 1
    assert np.array_equal(A.guard_page(), pages[3])


def test_f32_ties_are_midpoints():
    x = A.f32_bf16_ties(64)
    low = x.view(np.uint32) & 0xFFFF
    assert np.mean(low == 0x8000) > 0.2 and np.mean(low == 0x7FFF) > 0.2 and np.mean(low == 0x8001) > 0.2
