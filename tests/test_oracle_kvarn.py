"""Pins of the oracle's KVarN pieces: rotation, Sinkhorn balancing, page encoder, decode.

* the butterfly FWHT against scipy.linalg.hadamard (Sylvester construction) and the
  identities H H^T = 128 I, FWHT(FWHT(x)) = 128 x, FWHT(ones) = 128 e_0;
* Sinkhorn on rank-1 matrices of powers of two (closed form: c2 = b / mean(b)), on its
  transpose (rows and channels swap), and the balance invariant after the last step;
* the identity page X = I (closed form of every code and scale);
* page scaling by 2^k (codes and channel scales invariant, block scales x 2^k) and
  negation (codes and channel scales invariant, block scales negated);
* dequantization through the explicit matrix against the inverse butterfly, and the
  round-trip error bound of the whole page.
"""
import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle as O

H = hadamard(128).astype(np.float64)


def test_fwht_matches_sylvester_hadamard_columns():
    for j in range(128):
        e = np.zeros(128, np.float32)
        e[j] = 1.0
        assert np.array_equal(O.fwht128(e).astype(np.float64), H[:, j])
    assert np.array_equal(H @ H.T, 128 * np.eye(128))


def test_fwht_on_integers_and_involution():
    rng = np.random.default_rng(5)
    for _ in range(20):
        x = rng.integers(-100, 100, size=128).astype(np.float32)
        y = O.fwht128(x)
        assert np.array_equal(y.astype(np.float64), H @ x.astype(np.float64))
        assert np.array_equal(O.fwht128(y), 128 * x)
    assert np.array_equal(O.fwht128(np.ones(128, np.float32)), 128 * np.eye(128, dtype=np.float32)[0])


def test_sinkhorn_rank_one_closed_form_and_transpose():
    rng = np.random.default_rng(6)
    a = 2.0 ** rng.integers(-2, 4, size=128)          # token factors
    b = 2.0 ** rng.integers(-3, 3, size=128)          # channel factors
    A = np.outer(a, b).astype(np.float32)             # A[t][j] = a_t b_j, exact
    r2, c2 = O.sinkhorn128(A, 8)
    np.testing.assert_allclose(c2, b / b.mean(), rtol=4e-7)
    np.testing.assert_allclose(r2, a * b.mean(), rtol=4e-7)
    # transposing the matrix swaps the roles of tokens and channels
    r2t, c2t = O.sinkhorn128(np.ascontiguousarray(A.T), 8)
    np.testing.assert_allclose(c2t, a / a.mean(), rtol=4e-7)
    # converged after one iteration already
    r1, c1 = O.sinkhorn128(A, 1)
    np.testing.assert_allclose(c1, c2, rtol=4e-7)


def test_sinkhorn_balance_invariant_after_last_column_step():
    rng = np.random.default_rng(7)
    Y = rng.standard_t(3, size=(128, 128)).astype(np.float32) * (1 + 10 * (rng.random(128) < 0.05))
    A = (Y * Y).astype(np.float32)
    r2, c2 = O.sinkhorn128(A, 8)
    bal = (A.astype(np.float64) / (r2[:, None].astype(np.float64) * c2[None, :])).mean(axis=0)
    np.testing.assert_allclose(bal, 1.0, atol=1e-5)
    # more iterations balance the rows too (Sinkhorn's fixed point)
    r2, c2 = O.sinkhorn128(A, 200)
    rows = (A.astype(np.float64) / (r2[:, None].astype(np.float64) * c2[None, :])).mean(axis=1)
    np.testing.assert_allclose(rows, 1.0, atol=1e-3)


def test_sinkhorn_zero_rows_and_channels_are_guarded():
    A = np.zeros((128, 128), np.float32)
    A[:64, :32] = 4.0
    r2, c2 = O.sinkhorn128(A, 8)
    assert np.all(np.isfinite(r2)) and np.all(np.isfinite(c2))
    assert np.all(r2[64:] == 1.0) and np.all(c2[32:] == 1.0)


@pytest.mark.parametrize("N", (2, 3, 4, 5, 6, 8))
def test_identity_page_closed_form(N):
    X = np.full((128, 128), 0, np.uint16)
    X[np.arange(128), np.arange(128)] = 0x3F80                 # bf16 1.0
    codes, scales, cscale = O.encode_page_kvarn(N, X)
    assert np.all(cscale == 0x3C00)                            # A == 1 -> c = 1
    top = (1 << N) - 1
    for t in range(128):
        u = O.unpack_codes(N, codes[t])
        Y = H[t]                                               # FWHT(e_t) = column t = row t
        for b in range(4):
            seg = Y[32 * b: 32 * (b + 1)]
            d = O.f64_from_fp16(int(scales[t, b]))
            if np.all(seg == seg[0]):                          # constant block: all codes 0
                sigma = seg[0]
                assert d == -sigma * 2.0 ** -(N - 1)
                assert np.all(u[32 * b: 32 * (b + 1)] == 0)
            else:                                              # +1 -> code 0, -1 -> top
                assert d == -(2.0 ** -(N - 1))
                ub = u[32 * b: 32 * (b + 1)]
                assert np.all(ub[seg > 0] == 0) and np.all(ub[seg < 0] == top)


def _rand_page(rng, scale=1.0):
    x = (rng.standard_normal((128, 128)) * scale).astype(np.float32)
    x[:, rng.choice(128, 4, replace=False)] *= 15
    return O.canon_bf16(x)


@pytest.mark.parametrize("N", (2, 4, 8))
def test_page_scaling_and_negation(N):
    rng = np.random.default_rng(8 + N)
    X = _rand_page(rng)
    c0, s0, cs0 = O.encode_page_kvarn(N, X)
    Xf = X.astype(np.uint32) << 16
    for k in (-2, 3):
        Xk = ((Xf.view(np.float32) * np.float32(2.0 ** k)).view(np.uint32) >> 16).astype(np.uint16)
        c1, s1, cs1 = O.encode_page_kvarn(N, Xk)
        # A scales by 4^k, the token scales r2 absorb it (c2 starts at 1), so the channel
        # scales are unchanged and the block scales carry the 2^k
        assert np.array_equal(c0, c1) and np.array_equal(cs0, cs1)
        assert all(O.f64_from_fp16(int(a)) * 2.0 ** k == O.f64_from_fp16(int(b)) for a, b in zip(s0.ravel(), s1.ravel()))
    Xn = X ^ np.uint16(0x8000)
    c2, s2, cs2 = O.encode_page_kvarn(N, Xn)
    assert np.array_equal(c0, c2) and np.array_equal(cs0, cs2)
    assert np.array_equal(s2, np.where(s0 == 0, s0, s0 ^ np.uint16(0x8000)))


@pytest.mark.parametrize("N", (2, 3, 4, 5, 6, 8))
def test_page_roundtrip_bound_and_explicit_inverse(N):
    rng = np.random.default_rng(20 + N)
    X = _rand_page(rng, scale=0.7)
    codes, scales, cscale = O.encode_page_kvarn(N, X)
    xf = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Y = xf @ H.T                                   # rotation in binary64 (rows)
    off = 1 << (N - 1)
    for t in range(0, 128, 9):
        xh = O.dequant_token(O.KVARN2 + [2, 3, 4, 5, 6, 8].index(N), codes[t], scales[t], cscale)
        u = O.unpack_codes(N, codes[t]).astype(np.float64)
        c = np.array([O.f64_from_fp16(int(v)) for v in cscale])
        d = np.array([O.f64_from_fp16(int(v)) for v in scales[t]])
        Yh = c * np.repeat(d, 32) * (u - off)
        # explicit-matrix decode equals the inverse butterfly in binary64
        np.testing.assert_allclose(xh, (H @ Yh) / 128.0, rtol=0, atol=1e-12 * np.abs(Yh).max())
        # per-channel error in the rotated domain: at most one step (clamped code) plus
        # the rounding of W = Y / c in binary32
        err = np.abs(Y[t] - Yh)
        step = np.abs(c * np.repeat(d, 32))
        assert np.all(err <= step * (1 + 1e-6) + np.abs(Y[t]) * 2.0 ** -22)
        # and the value domain error is the same vector norm / sqrt(128)
        np.testing.assert_allclose(np.linalg.norm(xf[t] - xh), np.linalg.norm(Y[t] - Yh) / np.sqrt(128), rtol=1e-9)


def test_fwht_stage_order_rounding_example():
    """Stage order h = 1, 2, ..., 64 is part of the binary32 definition.  Hand-derived:
    x = (2^24, 1, 1, 0, 0, ...).  Stage h=1: (2^24+1 -> 2^24 (tie to even), 2^24-1, 1, 1);
    stage h=2: (2^24+1 -> 2^24, 2^24-1+1 = 2^24, 2^24-1, 2^24-2); later stages copy the
    four values with period 4.  The reverse stage order gives (2^24, 2^24-1, 2^24, 2^24-2)."""
    x = np.zeros(128, np.float32)
    x[0], x[1], x[2] = 2.0**24, 1.0, 1.0
    y = O.fwht128(x)
    ref = np.tile(np.array([2.0**24, 2.0**24, 2.0**24 - 1, 2.0**24 - 2], np.float32), 32)
    assert np.array_equal(y, ref)


def test_sinkhorn_matches_exact_iterates_and_iteration_count():
    """The binary32 Sinkhorn stays within 1e-5 of the same 8 iterations carried out in
    binary64 on a slowly converging matrix, and is far from 7 or 9 iterations."""
    rng = np.random.default_rng(17)
    A = np.ones((128, 128), np.float64)                 # block matrix that converges slowly
    A[:64, :64] = 9.0
    A[64:, 64:] = 9.0
    A[:8, 64:] = 81.0
    A *= 1 + 0.5 * rng.random((128, 128))
    A = A.astype(np.float32).astype(np.float64)

    def exact(iters):
        c2 = np.ones(128)
        for _ in range(iters):
            r2 = (A / c2[None, :]).mean(axis=1)
            c2 = (A / r2[:, None]).mean(axis=0)
        return c2

    _, c2 = O.sinkhorn128(A.astype(np.float32), 8)
    np.testing.assert_allclose(c2, exact(8), rtol=1e-5)
    for other in (7, 9):
        assert np.max(np.abs(exact(other) / exact(8) - 1)) > 1e-3
