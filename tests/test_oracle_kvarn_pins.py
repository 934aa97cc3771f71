"""Hand-derived binary32 pins of the KVarN page encoder's two branches that tolerance
checks cannot see ("Практическое руководство: запуск Bonsai-Ternary-27B на 120k токенах
с менее чем 10 ГБ VRAM", section "Как преобразование Уолша-Адамара и Sinkhorn спасают
качество при 4-битном сжатии": rotate, then pick a scale per dimension before quantizing).

1. The channel-scale guard.  A channel whose balanced mean square c2 lies in
   [FLT_MIN, 2^-50] has sqrt(c2) < 2^-25, which rounds to binary16 zero; the channel scale
   is then 1.0 (0x3C00).  The page below reaches that branch with ordinary bf16 values.

2. The order of the Sinkhorn sums and the reciprocal-then-multiply step.  A matrix whose
   row and column sums come out differently under a sequential sum (either direction), an
   adjacent-pair tree or a division in place of the reciprocal product, and exactly as
   stated under the halving tree `tree128` with reciprocals taken once per step.

Every expected value is derived in the docstrings from the definitions, not from the
oracle.  The checks are functions of the encoder/Sinkhorn callables so that the mutation
test can run them against oracles with planted mistakes.
"""
import numpy as np
import pytest

import oracle as O

BF16_ONE = 0x3F80


def _bf16_pow2(e: int, negative: bool = False) -> int:
    """bf16 bits of +-2^e (normal range)."""
    return (0x8000 if negative else 0) | ((e + 127) << 7)


def _fp16_pow2(e: int, negative: bool = False) -> int:
    """binary16 bits of +-2^e (normal range, -14 <= e <= 15)."""
    assert -14 <= e <= 15
    return (0x8000 if negative else 0) | ((e + 15) << 10)


def guard_page_scales():
    """Token t carries the factor s_t = sign_t * 2^e_t with e_t = t % 5 - 2 and a sign that
    flips every 5 tokens."""
    e = [t % 5 - 2 for t in range(128)]
    neg = [(t // 5) % 2 == 1 for t in range(128)]
    return e, neg


def guard_page() -> np.ndarray:
    """X[t][i] = s_t for i < 64, X[t][64] = s_t * 2^-40, X[t][i] = 0 for i > 64 (bf16)."""
    e, neg = guard_page_scales()
    X = np.zeros((128, 128), np.uint16)
    for t in range(128):
        X[t, :64] = _bf16_pow2(e[t], neg[t])
        X[t, 64] = _bf16_pow2(e[t] - 40, neg[t])
    return X


def check_guard_page(encode_page, N: int):
    """Derivation (binary32, every step exact unless said):
    rotation: the first 64 dims (all s) become 64s at dim 0 and exact zeros; the lone
      s*2^-40 at dim 64 spreads to s*2^-40 over dims 64..127 by the stages h < 64; stage
      h = 64 gives 64s + s*2^-40 -> 64s and 64s - s*2^-40 -> 64s (the tiny term is far below
      half an ulp), +s*2^-40 at dims 1..63 and -s*2^-40 at dims 65..127.
    squares: A[t][j] = 4096 s^2 at j in {0, 64}, s^2 * 2^-80 elsewhere (normal binary32).
    Sinkhorn, iteration 1: row sums with c2 = 1 absorb every tiny term into 8192 s^2, so
      r2 = 64 s^2 (a power of two, so 1/r2 is exact); column sums of A/r2 are 128 equal
      powers of two: c2 = 64 at j in {0, 64}, 2^-86 elsewhere (>= FLT_MIN, no row/column
      guard).  Iteration 2 finds A/c2 = 64 s^2 everywhere and reproduces both: fixed point.
    channel scales: sqrt(64) = 8 -> 0x4800; sqrt(2^-86) = 2^-43 rounds to binary16 zero
      -> guard -> 1.0 (0x3C00).  126 of the 128 channels take the guard.
    normalize: W = 8s at dims 0 and 64; +s*2^-40 on dims 1..63; -s*2^-40 on dims 65..127.
    E0, with off = 2^(N-1):
      blocks 0 and 2: signed max 8s -> d = 8s / -off = -sign(s) 2^(e+4-N) exactly; the 8s
        element -> t = -off -> code 0; the tiny ones -> t = +-off*2^-43 -> rint 0 -> off.
      blocks 1 and 3: constant +-s*2^-40 -> |d| <= 2^-38 -> binary16 zero -> d16 = +0 and
        every code off."""
    X = guard_page()
    e, neg = guard_page_scales()
    codes, scales, cscale = encode_page(N, X)
    want_c = np.full(128, 0x3C00, np.uint16)
    want_c[0] = want_c[64] = 0x4800
    assert np.array_equal(cscale, want_c), "channel scales %s" % cscale[:8]
    off = 1 << (N - 1)
    for t in range(128):
        d_big = _fp16_pow2(e[t] + 4 - N, negative=not neg[t])
        want_s = np.array([d_big, 0, d_big, 0], np.uint16)
        assert np.array_equal(scales[t], want_s), "token %d block scales %s" % (t, scales[t])
        u = O.unpack_codes(N, codes[t])
        want_u = np.full(128, off, np.uint8)
        want_u[0] = want_u[64] = 0
        assert np.array_equal(u, want_u), "token %d codes" % t


@pytest.mark.parametrize("N", (2, 3, 4, 5, 6, 8))
def test_channel_scale_guard_page(N):
    check_guard_page(O.encode_page_kvarn, N)


def order_matrix() -> np.ndarray:
    """A 128x128 matrix of non-negative binary32 values (zero where not listed):
    row 0: 3 everywhere except A[0][5] = 5, A[0][6] = 1, A[0][7] = 12 and
           A[0][100] = A[0][101] = A[0][110] = 0 (row sum 122*3 + 18 = 384);
    row 1: A[1][0] = 1, A[1][1] = 2^24, A[1][64] = 1;
    rows 8 and 72: A[.][100] = 2^-17, A[.][101] = 128;
    row 9: A[9][100] = 1;
    rows 20, 21, 22: A[20][110] = 5, A[21][110] = A[22][110] = 1."""
    A = np.zeros((128, 128), np.float32)
    A[0, :] = 3.0
    A[0, 5], A[0, 6], A[0, 7] = 5.0, 1.0, 12.0
    A[0, 100] = A[0, 101] = A[0, 110] = 0.0
    A[1, 0], A[1, 1], A[1, 64] = 1.0, 2.0 ** 24, 1.0
    for t in (8, 72):
        A[t, 100], A[t, 101] = 2.0 ** -17, 128.0
    A[9, 100] = 1.0
    A[20, 110], A[21, 110], A[22, 110] = 5.0, 1.0, 1.0
    return A


def check_sinkhorn_order(sinkhorn):
    """One iteration (row step with c2 = 1, then column step), and one row of a second
    row step, derived by hand:
    r2[0] = 384/128 = 3 (integer partial sums, exact).
    r2[1]: tree128 pairs (0, 64) first: 1 + 1 = 2, meets 2^24 only at the last level:
      2^24 + 2 (exact) -> r2 = 2^17 + 2^-6.  A sequential sum either way, or an adjacent-
      pair tree, adds a lone 1 to 2^24 first (a tie, rounded to even 2^24): r2 = 2^17.
    r2[8] = r2[72]: 128 + 2^-17 is a tie at half an ulp of 128, rounded to even 128: r2 = 1.
    r2[9] = 1/128; every all-zero row takes the guard (r2 = 1).
    c2[5]: the only nonzero term is A[0][5] * (1/r2[0]) = 5 * fl(1/3);
      fl(1/3) = 11184811 * 2^-25, times 5 = 55924055 * 2^-25 -> 13981014 * 2^-23 (the two
      dropped bits are 0b11, rounded up), so c2[5] = 13981014 * 2^-30.  The division
      5 / 3 would give 13981013 * 2^-23 instead.
    c2[100]: terms 2^-17 (t = 8), 2^-17 (t = 72), 128 (t = 9: 1 * 2^7).  tree128 adds
      t = 8 and t = 72 first (2^-16), then 128 + 2^-16 exactly at the last level:
      c2 = 1 + 2^-23.  Sequential sums and adjacent pairs add a lone 2^-17 to 128 first
      (a tie, to even 128): c2 = 1.
    c2[110]: r2[20] = 5 * 2^-7, fl(1/r2[20]) = fl(25.6) = 13421773 * 2^-19, times 5 =
      67108865 * 2^-19 -> 128 exactly; rows 21 and 22 give 128 each: c2[110] = 3.
    Iteration 2, row 20 (its only term is in column 110): r2[20] = 5 * fl(1/3) / 128 =
      13981014 * 2^-30, where a division 5 / 3 gives 13981013 * 2^-30."""
    A = order_matrix()
    r2, c2 = sinkhorn(A, 1)
    assert float(r2[0]) == 3.0
    assert float(r2[1]) == 2.0 ** 17 + 2.0 ** -6, "row sum order: r2[1] = %r" % float(r2[1])
    assert float(r2[8]) == 1.0 and float(r2[72]) == 1.0
    assert float(r2[9]) == 2.0 ** -7
    assert all(float(r2[t]) == 1.0 for t in range(128) if t not in (0, 1, 8, 9, 20, 21, 22, 72))
    assert float(c2[5]) == 13981014 * 2.0 ** -30, "reciprocal step: c2[5] = %r" % float(c2[5])
    assert float(c2[100]) == 1.0 + 2.0 ** -23, "column sum order: c2[100] = %r" % float(c2[100])
    assert float(r2[20]) == 5.0 * 2.0 ** -7 and float(c2[110]) == 3.0
    r2, c2 = sinkhorn(A, 2)
    assert float(r2[20]) == 13981014 * 2.0 ** -30, "row reciprocal step: r2[20] = %r" % float(r2[20])


def test_sinkhorn_sum_order_and_reciprocal_step():
    check_sinkhorn_order(O.sinkhorn128)
