"""Pins of the oracle's var-norm over affine bases (kvarnN_1: KVarN with qN_1 as the inner
quantizer).

* The rotation, Sinkhorn balancing and channel scales are those of kvarnN on the same page
  (only the inner quantizer differs), so the channel-scale rows are identical.
* The inner codes and {step, minimum} scales equal the (separately pinned) affine block
  quantizer applied to W = FWHT(x) * (1 / c) in binary32, with the (separately pinned)
  butterfly FWHT: the composition the page encoder defines.
* Decode through the explicit Hadamard matrix equals the oracle's inverse, and the
  round-trip error in the rotated domain is at most half a step per channel plus the
  binary32 rounding of W (affine codes round to nearest); the value-domain error is that
  vector norm over sqrt(128).
* The stream API: granule 128, 16-byte scale rows, one channel-scale row per page.
"""
import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle as O

H = hadamard(128).astype(np.float64)
NS = (2, 3, 4, 5, 6, 8)


def _fmt(N):
    return O.KVARN2_1 + NS.index(N)


def _page(rng, scale=0.7):
    x = (rng.standard_normal((128, 128)) * scale).astype(np.float32)
    x[:, rng.choice(128, 4, replace=False)] *= 15
    return O.canon_bf16(x)


@pytest.mark.parametrize("N", NS)
def test_channel_scales_match_kvarn_and_inner_is_affine(N):
    rng = np.random.default_rng(40 + N)
    X = _page(rng)
    _, _, c0 = O.encode_page_kvarn(N, X)
    codes, scales, c1 = O.encode_page_kvarn(N, X, affine=True)
    assert np.array_equal(c0, c1)
    ic = (np.float32(1.0) / np.array([O.f64_from_fp16(int(v)) for v in c1], np.float32)).astype(np.float32)
    for t in range(0, 128, 7):
        xf = (X[t].astype(np.uint32) << 16).view(np.float32)
        W = (O.fwht128(xf) * ic).astype(np.float32)
        u = O.unpack_codes(N, codes[t])
        for b in range(4):
            d, m, ub = O.encode_block_q1(N, W[32 * b: 32 * (b + 1)])
            assert (d, m) == (int(scales[t, 2 * b]), int(scales[t, 2 * b + 1]))
            assert np.array_equal(ub, u[32 * b: 32 * (b + 1)])


@pytest.mark.parametrize("N", (2, 4, 8))
def test_roundtrip_bound_and_explicit_inverse(N):
    rng = np.random.default_rng(60 + N)
    X = _page(rng)
    codes, scales, cscale = O.encode_page_kvarn(N, X, affine=True)
    xf = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Y = xf @ H.T
    c = np.array([O.f64_from_fp16(int(v)) for v in cscale])
    for t in range(0, 128, 11):
        xh = O.dequant_token(_fmt(N), codes[t], scales[t], cscale)
        u = O.unpack_codes(N, codes[t]).astype(np.float64)
        d = np.array([O.f64_from_fp16(int(scales[t, 2 * b])) for b in range(4)])
        m = np.array([O.f64_from_fp16(int(scales[t, 2 * b + 1])) for b in range(4)])
        Yh = c * (np.repeat(m, 32) + np.repeat(d, 32) * u)
        np.testing.assert_allclose(xh, (H @ Yh) / 128.0, rtol=0, atol=1e-12 * np.abs(Yh).max())
        # half a step per channel, plus the binary16 rounding of the minimum and step
        # (relative 2^-11 of |m| and of the top code's value) and the binary32 W
        step = np.abs(c * np.repeat(d, 32))
        slack = np.abs(c) * (np.repeat(np.abs(m), 32) + np.repeat(np.abs(d), 32) * ((1 << N) - 1)) * 2.0 ** -10
        err = np.abs(Y[t] - Yh)
        assert np.all(err <= 0.5 * step + slack + np.abs(Y[t]) * 2.0 ** -20)
        np.testing.assert_allclose(np.linalg.norm(xf[t] - xh), np.linalg.norm(Y[t] - Yh) / np.sqrt(128), rtol=1e-9)


def test_stream_api():
    f = O.KVARN4_1
    N, kind, cb, sb, pb = O.format_info(f)
    assert (N, kind, cb, sb, pb) == (4, O.KIND_KVARN1, 64, 16, 256)
    assert O.granule(f, O.Q4_0) == 128 and O.granule(O.Q4_0, f) == 128
    rng = np.random.default_rng(1)
    x = np.concatenate([_page(rng), _page(rng)])
    codes, scales, cs = O.encode_stream(f, 256, x)
    assert codes.shape == (256, 64) and scales.shape == (256, 8) and cs.shape == (2, 128)
    c2, s2, cs2 = O.encode_page_kvarn(4, x[128:], affine=True)
    assert np.array_equal(codes[128:], c2) and np.array_equal(scales[128:], s2) and np.array_equal(cs[1], cs2)
    with pytest.raises(ValueError):
        O.encode_stream(f, 100, x)
