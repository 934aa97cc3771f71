"""Pins of the oracle's causal prefill attention over the mixed cache.

  * Brute force with numpy and scipy's softmax: every query i of the chunk attends to the
    tokens 0 .. n - n_new + i as the cache holds them (rows below n_q dequantized from the
    encoding of the whole quantized region, exact bf16 rows after), for chunks that lie in
    the tail, straddle the boundary, or lie wholly in the quantized region (including a
    KVarN page only partly visible to the first queries).
  * The last query of a chunk sees the whole sequence, so it equals the decode attention
    over all n tokens; a chunk of one token is decode.
  * n_new == 0 is an error.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle as O

SIGMA = 1.0 / np.sqrt(128)


def _rows(rng, n):
    x = rng.standard_normal((n, 128)).astype(np.float32)
    x[:, [5, 66]] *= 10.0
    return O.canon_bf16(x)


def _vals(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _run(fmt_k, fmt_v, n, n_q, n_new, seed):
    rng = np.random.default_rng(seed)
    k, v = _rows(rng, n), _rows(rng, n)
    q = rng.standard_normal((n_new, 4, 128))
    kq = O.encode_stream(fmt_k, n_q, k) if n_q else None
    vq = O.encode_stream(fmt_v, n_q, v) if n_q else None
    got = O.prefill_attention(n, n_q, n_new, fmt_k, fmt_v, kq, vq, k[n_q:], v[n_q:], q, SIGMA)
    return k, v, q, kq, vq, got


@pytest.mark.parametrize("fmt_k,fmt_v", [(O.Q4_0, O.Q4_0), (O.Q3_1, O.KVARN4), (O.KVARN2, O.Q8_0)])
@pytest.mark.parametrize("n,n_q,n_new", [(400, 200, 64), (400, 384, 100), (700, 640, 300)])
def test_brute_force(fmt_k, fmt_v, n, n_q, n_new):
    if O.granule(fmt_k, fmt_v) == 128 and n_q % 128:
        n_q -= n_q % 128
    k, v, q, kq, vq, got = _run(fmt_k, fmt_v, n, n_q, n_new, 11 + n + n_q)
    K, V = _vals(k), _vals(v)
    if n_q:
        K[:n_q] = O.dequant_stream(fmt_k, n_q, *kq)
        V[:n_q] = O.dequant_stream(fmt_v, n_q, *vq)
    for i in range(n_new):
        ctx = n - n_new + i + 1
        for h in range(4):
            p = softmax(SIGMA * (K[:ctx] @ q[i, h]))
            np.testing.assert_allclose(got[i, h], p @ V[:ctx], rtol=1e-10, atol=1e-12)


def test_last_query_is_decode_and_single_token_chunk():
    n, n_q = 500, 256
    k, v, q, kq, vq, got = _run(O.KVARN4, O.KVARN4, n, n_q, 37, 5)
    dec = O.attention(n, n_q, O.KVARN4, O.KVARN4, kq, vq, k[n_q:], v[n_q:], q[-1], SIGMA)
    np.testing.assert_allclose(got[-1], dec, rtol=1e-12, atol=1e-14)
    one = O.prefill_attention(n, n_q, 1, O.KVARN4, O.KVARN4, kq, vq, k[n_q:], v[n_q:], q[-1:], SIGMA)
    np.testing.assert_allclose(one[0], dec, rtol=1e-12, atol=1e-14)


def test_empty_chunk_is_an_error():
    with pytest.raises(ValueError):
        O.prefill_attention(10, 0, 0, O.Q4_0, O.Q4_0, None, None, np.zeros((10, 128), np.uint16),
                            np.zeros((10, 128), np.uint16), np.zeros((0, 4, 128)), SIGMA)
