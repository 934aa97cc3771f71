"""Pins of the oracle's attention-fidelity measure (KL divergence of the attention
distribution over the cache's keys from the one over the exact keys).

  * scipy's relative entropy (scipy.stats.entropy) of the two softmax distributions, built
    here with numpy from the exact bf16 keys and the oracle's dequantized rows, equals the
    oracle's value for every format family, with and without a tail; so does the same
    with the roles of P and Q swapped only when the two are equal (KL is asymmetric, and
    a swapped implementation fails the first check);
  * an all-exact cache (tail >= n, or the bf16 format) has KL exactly 0;
  * KL >= 0 for every tail length, and 0 once the tail holds every token (it is not
    monotone in the tail: making some keys exact can undo errors that partly cancelled);
  * n == 0 is an error.
"""
import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import entropy

import oracle as O

SIGMA = 1.0 / np.sqrt(128)


def _rows(rng, n, outliers=True):
    x = rng.standard_normal((n, 128)).astype(np.float32)
    if outliers:
        x[:, [3, 40, 77, 101]] *= 15.0
    return O.canon_bf16(x)


def _values(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _kld_by_scipy(fmt, n, n_q, rows, q):
    K = _values(rows[:n]).copy()
    if n_q:
        c, s, cs = O.encode_stream(fmt, n_q, rows)
        K[:n_q] = O.dequant_stream(fmt, n_q, c, s, cs)
    E = _values(rows[:n])
    out = []
    for h in range(q.shape[0]):
        P = softmax(SIGMA * (E @ q[h]))
        Q = softmax(SIGMA * (K @ q[h]))
        out.append(entropy(P, Q))
    return np.array(out)


def _kld(fmt, n, n_q, rows, q):
    kq = O.encode_stream(fmt, n_q, rows) if n_q else None
    return O.attention_kld(n, n_q, fmt, kq, rows[:n], q, SIGMA)


@pytest.mark.parametrize("fmt", [O.Q2_0, O.Q3_1, O.Q4_0, O.Q8_0, O.KVARN2, O.KVARN4])
@pytest.mark.parametrize("n,n_q", [(300, 300), (300, 256), (513, 384)])
def test_matches_scipy_relative_entropy(fmt, n, n_q):
    if O.granule(fmt, fmt) == 128 and n_q % 128:
        pytest.skip("kvarn boundaries are page multiples")
    rng = np.random.default_rng(1000 + 7 * fmt + n_q)
    rows = _rows(rng, n)
    q = rng.standard_normal((4, 128))
    got = _kld(fmt, n, n_q, rows, q)
    ref = _kld_by_scipy(fmt, n, n_q, rows, q)
    assert np.all(ref > 0)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-15)


def test_exact_cache_has_zero_divergence():
    rng = np.random.default_rng(5)
    rows = _rows(rng, 200)
    q = rng.standard_normal((4, 128))
    assert np.all(_kld(O.Q4_0, 200, 0, rows, q) == 0.0)          # everything in the tail
    assert np.all(_kld(O.BF16, 200, 200, rows, q) == 0.0)        # bf16 "quantized" rows


def test_nonnegative_and_zero_at_full_tail():
    rng = np.random.default_rng(9)
    n = 1024
    rows = _rows(rng, n)
    q = 3.0 * rng.standard_normal((4, 128))                      # peaked attention
    for fmt in (O.Q2_0, O.Q3_0, O.KVARN3):
        G = O.granule(fmt, fmt)
        for tail in (0, 128, 256, 512, 1024):
            n_q = O.nq_after(0, n, tail, G)
            k = _kld(fmt, n, n_q, rows, q)
            assert np.all(k >= 0.0)
        assert np.all(k == 0.0)


def test_empty_is_an_error():
    with pytest.raises(ValueError):
        O.attention_kld(0, 0, O.Q4_0, None, np.zeros((1, 128), np.uint16), np.zeros((4, 128)), SIGMA)
