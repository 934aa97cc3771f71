"""Pins of the oracle's precision-tail state machine and its binary64 attention.

State machine: ring capacity and the quantized boundary n_q against hand-worked cases
(the page example "tail 1024, positions 0..N-1024 quantized") and the invariants that
occupancy never exceeds T + G - 1, stays at least min(n, T) while only appends happen,
and n_q never decreases.

Attention: n = 1 gives v_0; identical keys or q = 0 give the mean of the values;
brute force with mpmath at 50 digits on tiny contexts; a full-precision tail
(T >= n) equals scipy's softmax over the bf16 values; tail = 0 equals attention over
directly encoded tokens.
"""
import mpmath
import numpy as np
import pytest
from scipy.special import softmax

import oracle as O


def test_ring_capacity_and_granule():
    assert O.granule(O.Q4_0, O.Q4_0) == 1
    assert O.granule(O.KVARN4, O.KVARN4) == 128
    assert O.granule(O.Q4_0, O.KVARN3) == 128
    assert O.ring_capacity(0, 1) == 0
    assert O.ring_capacity(1024, 1) == 1024
    assert O.ring_capacity(1024, 128) == 1152          # T + G - 1 = 1151 -> next page
    assert O.ring_capacity(2048, 128) == 2176
    assert O.ring_capacity(0, 128) == 128


def test_nq_page_example():
    # "tail = 1024 with main format q3_0: the last 1024 tokens stay high precision,
    # positions 0 .. N-1024 are q3_0" -- for N = 5000 tokens, n_q = 3976.
    assert O.nq_after(0, 5000, 1024, 1) == 3976
    assert O.nq_after(0, 1000, 1024, 1) == 0
    assert O.nq_after(0, 5000, 1024, 128) == 3968        # page-rounded down
    assert O.nq_after(4000, 5000, 1024, 1) == 4000        # never decreases
    assert O.nq_after(0, 5000, 0, 1) == 5000              # tail 0 -> everything quantized


def test_state_machine_invariants_random_walk():
    rng = np.random.default_rng(3)
    for G in (1, 128):
        for T in (0, 1, 256, 1024):
            R = O.ring_capacity(T, G)
            for with_spills in (False, True):
                n = nq = 0
                for _ in range(300):
                    if not with_spills or rng.random() < 0.85:
                        n += int(rng.integers(1, 700))
                        new = O.nq_after(nq, n, T, G)
                    else:
                        keep = int(rng.integers(0, T + 1))
                        new = O.nq_after(nq, n, keep, G)
                    assert new >= nq and new % G == 0 and new <= n
                    nq = new
                    occ = n - nq
                    # the ring never holds more than T + G - 1 tokens ...
                    assert occ <= T + G - 1 and occ <= R
                    # ... and, with appends only, always the last min(n, T) tokens
                    if not with_spills:
                        assert occ >= min(n, T)


def test_ring_image_slots():
    x = np.arange(10 * 128, dtype=np.uint16).reshape(10, 128)
    ring = O.ring_image(10, 6, 4, x)
    for p in range(6, 10):
        assert np.array_equal(ring[p % 4], x[p])


def _attn_inputs(rng, n, fmt, g=4, scale=1.0):
    k = O.canon_bf16((rng.standard_normal((n, 128)) * scale).astype(np.float32))
    v = O.canon_bf16(rng.standard_normal((n, 128)).astype(np.float32))
    q = rng.standard_normal((g, 128))
    return k, v, q


def _bf(x):
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("fmt", [O.Q4_0, O.Q2_1, O.BF16])
def test_attention_n1_and_identical_keys(fmt):
    rng = np.random.default_rng(11)
    k, v, q = _attn_inputs(rng, 1, fmt)
    kq = O.encode_stream(fmt, 1, k)
    vq = O.encode_stream(fmt, 1, v)
    out = O.attention(1, 1, fmt, fmt, kq, vq, None, None, q, 0.088)
    v0 = O.dequant_stream(fmt, 1, *vq)[0]
    assert np.array_equal(out, np.tile(v0, (4, 1)))
    # identical keys: uniform weights -> mean of the values
    n = 37
    kk = np.tile(k, (n, 1))
    _, v, _ = _attn_inputs(rng, n, fmt)
    kq = O.encode_stream(fmt, n, kk)
    vq = O.encode_stream(fmt, n, v)
    out = O.attention(n, n, fmt, fmt, kq, vq, None, None, q, 0.088)
    vm = O.dequant_stream(fmt, n, *vq).mean(axis=0)
    np.testing.assert_allclose(out, np.tile(vm, (4, 1)), rtol=1e-13, atol=1e-15)
    # q = 0: the same mean for any keys
    k, v, _ = _attn_inputs(rng, n, fmt)
    kq = O.encode_stream(fmt, n, k)
    vq = O.encode_stream(fmt, n, v)
    out = O.attention(n, n, fmt, fmt, kq, vq, None, None, np.zeros((2, 128)), 0.088)
    np.testing.assert_allclose(out, np.tile(O.dequant_stream(fmt, n, *vq).mean(axis=0), (2, 1)), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("n,nq,fmt", [(3, 2, O.Q4_0), (16, 16, O.Q3_1), (11, 0, O.Q8_0), (16, 5, O.Q6_0)])
def test_attention_brute_force_mpmath(n, nq, fmt):
    rng = np.random.default_rng(100 + n)
    k, v, q = _attn_inputs(rng, n, fmt, g=2, scale=3.0)
    kq = O.encode_stream(fmt, nq, k)
    vq = O.encode_stream(fmt, nq, v)
    sigma = 0.125
    out = O.attention(n, nq, fmt, fmt, kq, vq, k[nq:], v[nq:], q, sigma)
    K = np.vstack([O.dequant_stream(fmt, nq, *kq), _bf(k[nq:])]) if nq else _bf(k)
    V = np.vstack([O.dequant_stream(fmt, nq, *vq), _bf(v[nq:])]) if nq else _bf(v)
    mpmath.mp.dps = 50
    for h in range(2):
        s = [mpmath.mpf(sigma) * mpmath.fsum(mpmath.mpf(float(q[h, i])) * mpmath.mpf(float(K[t, i]))
                                             for i in range(128)) for t in range(n)]
        e = [mpmath.exp(st) for st in s]
        den = mpmath.fsum(e)
        for i in range(0, 128, 7):
            ref = mpmath.fsum(e[t] * mpmath.mpf(float(V[t, i])) for t in range(n)) / den
            assert abs(out[h, i] - float(ref)) <= 1e-12 * max(1.0, abs(float(ref)))


def test_full_tail_equals_softmax_over_bf16():
    rng = np.random.default_rng(12)
    n = 300
    k, v, q = _attn_inputs(rng, n, O.Q4_0, g=4)
    out = O.attention(n, 0, O.Q2_0, O.Q2_0, (None, None, None), (None, None, None), k, v, q, 0.09)
    K, V = _bf(k), _bf(v)
    ref = softmax(0.09 * (q @ K.T), axis=1) @ V
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_empty_context_is_an_error():
    with pytest.raises(ValueError):
        O.attention(0, 0, O.Q4_0, O.Q4_0, (None, None, None), (None, None, None), None, None,
                    np.zeros((1, 128)), 1.0)
