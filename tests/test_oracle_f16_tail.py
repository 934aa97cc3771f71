"""Pins of the oracle's F16-tail mode (binary16 as the canonical 16-bit type).

  * The vectorized canonicalization equals the oracle's scalar saturating conversion
    (itself pinned against numpy) on random values over many binades and on the edges:
    +-65504 and beyond, the subnormal range, ties, signed zeros.
  * Values exact in both bf16 and binary16 encode to the same codes in both modes, for
    every format family (the encoders see the same floats).
  * With every token in the tail, attention equals scipy's softmax over the binary16 values;
    the mode is process-wide and the context manager restores it.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle as O

SIGMA = 1.0 / np.sqrt(128)


def test_vectorized_matches_scalar():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 20, 20000))).astype(np.float32)
    edges = np.array([0.0, -0.0, 65504, -65504, 65519.99, 65520, 1e30, -1e30, 2.0 ** -24, 2.0 ** -25,
                      -(2.0 ** -25), 3 * 2.0 ** -26, 2.0 ** -14, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11],
                     np.float32)
    x = np.concatenate([x, edges])
    got = O.canon_f16(x)
    ref = np.array([O.fp16s_from_f32(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", [O.Q2_0, O.Q3_1, O.Q4_0, O.Q6_1, O.Q8_0])
def test_modes_agree_on_values_exact_in_both(fmt):
    rng = np.random.default_rng(fmt)
    vals = (rng.integers(-64, 65, (4, 128)) / 4.0).astype(np.float32)     # exact in bf16 and f16
    b = O.canon_bf16(vals)
    with O.canonical("f16"):
        h = O.canon(vals)
        enc_h = [O.encode_token(fmt, h[t]) for t in range(4)]
    enc_b = [O.encode_token(fmt, b[t]) for t in range(4)]
    for (cb, sb), (ch, sh) in zip(enc_b, enc_h):
        assert np.array_equal(cb, ch) and np.array_equal(sb, sh)


def test_kvarn_page_modes_agree():
    rng = np.random.default_rng(11)
    vals = (rng.integers(-64, 65, (128, 128)) / 4.0).astype(np.float32)
    pb = O.encode_page_kvarn(4, O.canon_bf16(vals))
    with O.canonical("f16"):
        ph = O.encode_page_kvarn(4, O.canon(vals))
    for a, b in zip(pb, ph):
        assert np.array_equal(a, b)


def test_full_tail_attention_over_binary16_values():
    rng = np.random.default_rng(5)
    n = 300
    x = (rng.standard_normal((2, n, 128)) * 3).astype(np.float32)
    q = rng.standard_normal((4, 128))
    with O.canonical("f16"):
        k, v = O.canon(x[0]), O.canon(x[1])
        out = O.attention(n, 0, O.Q4_0, O.Q4_0, (None, None, None), (None, None, None), k, v, q, SIGMA)
    assert not O.canonical_f16()
    K, V = k.view(np.float16).astype(np.float64), v.view(np.float16).astype(np.float64)
    for h in range(4):
        np.testing.assert_allclose(out[h], softmax(SIGMA * (K @ q[h])) @ V, rtol=1e-12, atol=1e-14)
