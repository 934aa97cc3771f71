"""Crafted K/V inputs for the edge-case parity tests, as bf16 bit patterns (uint16) or
float32 values.  Pure input construction: no step of the cache method is computed here;
both the HIP path and the oracle are fed these same arrays.

* block_catalog(N): 32-value blocks, every value exact in bf16, aimed at the branches of
  the block encoders for N-bit codes: all-zero and constant blocks, tied extremes (+a and
  -a), values on exact rounding ties of x / d for the scales the signed maximum (qN_0) or
  the range (qN_1) give, scales in the binary16 subnormal range (one on a rounding tie),
  scales that round to binary16 zero, saturated scales (|x| up to 2^30), bf16 subnormal
  inputs, minima beyond binary16 range, an isolated outlier, alternating signs.
* crafted_rows(N, n, salt): n tokens built from the catalog (4 blocks each, a rotating
  choice, signs flipped per sweep).
* crafted_pages(): 128-token pages for the KVarN encoder: zero, constant, identity, the
  channel-guard page, huge (|x| ~ 2^30) and bf16-subnormal pages, a page with one token, a
  page with one 2^20 outlier token, a page mixing tiny and unit tokens.
* f32_bf16_ties(n, seed): float32 inputs on, and next to, the midpoints between bf16
  values (round to nearest even decides).
"""
from __future__ import annotations

import numpy as np


def bf16_bits(x) -> np.ndarray:
    """float32 values that are exact in bf16 -> their bf16 bits (asserts exactness)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def _odd_grid(n, lo, hi):
    """n odd integers cycling over [lo, hi] (|value| <= 255 keeps 8 significant bits)."""
    vals = np.arange(lo, hi + 1)
    vals = vals[(vals % 2) != 0]
    return vals[np.arange(n) % len(vals)]


def block_catalog(N: int) -> list:
    off = 1 << (N - 1)
    top = (1 << N) - 1
    B = []
    f = lambda v: np.asarray(v, dtype=np.float64).astype(np.float32)
    B.append(np.zeros(32, np.float32))                                   # all zero
    for c in (1.5, -1.5, 2.0 ** -30, -3 * 2.0 ** 20):                   # constant blocks
        B.append(np.full(32, c, np.float32))
    x = f(np.linspace(-2.75, 2.75, 32) // 0.25 * 0.25)                    # tied extremes
    x[0], x[1] = 3.0, -3.0
    B.append(x)
    y = x.copy()
    y[1] = -3.015625                                                      # |min| one bf16 step above max
    B.append(y)
    k = -3
    # qN_0 ties: signed maximum -off 2^k (d = +2^k) or +off 2^k (d = -2^k); the other values
    # (j + 1/2) 2^k for j in [-off, off - 1], as odd multiples of 2^(k-1)
    for sgn in (-1.0, 1.0):
        j2 = _odd_grid(31, -min(2 * off - 1, 255), min(2 * off - 1, 255))
        x = np.concatenate([[sgn * off * 2.0 ** k], j2 * 2.0 ** (k - 1)])
        B.append(f(x))
    # qN_1 ties: minimum 0, maximum (2^N - 1) 2^k (step exactly 2^k), values (j + 1/2) 2^k
    j2 = _odd_grid(30, 1, min(2 * top - 1, 255))
    B.append(f(np.concatenate([[0.0, top * 2.0 ** k], j2 * 2.0 ** (k - 1)])))
    B.append(f(np.arange(32) - 16.0))                                    # worked example
    # binary16 subnormal scales: |m| / off = 5 * 2^-20 (exact), and 33 * 2^-25 (a tie of the
    # binary16 rounding, quantum 2^-24)
    c = np.array([5, 4.5, -3, 1.25, -4.75, 0.5, 2, -1] * 4, np.float64)
    B.append(f(-off * 2.0 ** -20 * c))
    t = np.array([33, 17, -20, 5, -32, 1, 9, -12] * 4, np.float64)
    B.append(f(-off * 2.0 ** -25 * t))
    B.append(f(np.array([1, -3, 2, 3, -1, 0, -2, 1] * 4) * 2.0 ** -30))  # scale -> binary16 zero
    # saturated scales: signed maximum 2^30, -off 2^16, 65280 off (exact binary16)
    B.append(f(np.concatenate([[2.0 ** 30], [(-1) ** i * 2.0 ** (i % 30) for i in range(31)]])))
    B.append(f(np.concatenate([[-off * 2.0 ** 16], np.linspace(-100, 100, 31).round()])))
    B.append(f(np.concatenate([[65280.0 * off], np.arange(31) * 256.0 - 4096.0])))
    # bf16 subnormal inputs
    B.append(f(np.array([2.0 ** -126, -2.0 ** -130, 2.0 ** -133, 0.0, -2.0 ** -127, 2.0 ** -131, 2.0 ** -129, -2.0 ** -128] * 4)))
    # minimum beyond binary16 range (affine minimum saturates)
    B.append(f(np.concatenate([[-2.0 ** 17, 0.0], np.linspace(-2.0 ** 17, 0, 30).round(-12)])))
    x = np.ones(32, np.float64)
    x[7] = 2.0 ** 20                                                      # isolated outlier
    B.append(f(x))
    B.append(f(np.array([1.0, -1.0] * 16)))                              # alternating signs
    for b in B:
        bf16_bits(b)                                                      # all exact in bf16
    return B


def crafted_rows(N: int, n: int, salt: int = 0, max_abs: float | None = None,
                 min_abs: float | None = None) -> np.ndarray:
    """[n][128] bf16 bits: token t, block b = catalog[(3 t + b + salt) % L], sign flipped
    on odd sweeps.  max_abs drops catalog blocks with larger values, min_abs nonzero blocks
    whose largest |x| is smaller."""
    cat = block_catalog(N)
    if max_abs is not None:
        cat = [b for b in cat if np.abs(b).max() <= max_abs]
    if min_abs is not None:
        cat = [b for b in cat if np.abs(b).max() == 0 or np.abs(b).max() >= min_abs]
    L = len(cat)
    rows = np.empty((n, 128), np.float32)
    for t in range(n):
        for b in range(4):
            i = 3 * t + b + salt
            v = cat[i % L]
            rows[t, 32 * b:32 * (b + 1)] = -v if (i // L) % 2 else v
    return bf16_bits(rows)


def guard_page() -> np.ndarray:
    """X[t][i] = s_t (i < 64), s_t 2^-40 (i = 64), 0 elsewhere; s_t = +-2^(t % 5 - 2), the
    sign flipping every 5 tokens: 126 of the 128 balanced channel scales underflow binary16."""
    X = np.zeros((128, 128), np.float32)
    for t in range(128):
        s = (-1.0 if (t // 5) % 2 else 1.0) * 2.0 ** (t % 5 - 2)
        X[t, :64] = s
        X[t, 64] = s * 2.0 ** -40
    return bf16_bits(X)


def crafted_pages(seed: int = 7) -> list:
    rng = np.random.default_rng(seed)
    pages = []
    pages.append(np.zeros((128, 128), np.float32))                       # zero page
    pages.append(np.full((128, 128), 1.5, np.float32))                    # constant page
    pages.append(np.eye(128, dtype=np.float32))                           # identity page
    g = guard_page()
    pages.append((g.astype(np.uint32) << 16).view(np.float32))
    h = rng.integers(-4, 5, size=(128, 128)).astype(np.float32) * np.float32(2.0 ** 28)
    pages.append(h)                                                       # |x| up to 2^30
    s = rng.integers(-3, 4, size=(128, 128)).astype(np.float32) * np.float32(2.0 ** -132)
    pages.append(s)                                                       # bf16 subnormals
    one = np.zeros((128, 128), np.float32)
    one[37] = rng.integers(-8, 9, size=128) * 0.25
    pages.append(one)                                                     # a single token
    o = (rng.integers(-8, 9, size=(128, 128)) * 0.25).astype(np.float32)
    o[90] *= np.float32(2.0 ** 20)
    pages.append(o)                                                       # one outlier token
    m = (rng.integers(-8, 9, size=(128, 128)) * 0.25).astype(np.float32)
    m[::2] *= np.float32(2.0 ** -60)
    pages.append(m)                                                       # tiny and unit tokens
    return [bf16_bits(p) for p in pages]


def f32_bf16_ties(n: int, seed: int = 3) -> np.ndarray:
    """[n][128] float32: bf16 values (random exponents near 1), each element moved to the
    midpoint above it (a tie), one float32 step below or above that midpoint, or left on
    the bf16 value."""
    rng = np.random.default_rng(seed)
    hi = rng.integers(0x3E00, 0x4100, size=(n, 128)).astype(np.uint32)
    hi |= (rng.integers(0, 2, size=(n, 128)).astype(np.uint32) << 15)    # random sign
    kind = rng.integers(0, 4, size=(n, 128))
    low = np.choose(kind, [np.uint32(0x8000), np.uint32(0x7FFF), np.uint32(0x8001), np.uint32(0)])
    return ((hi << 16) | low).astype(np.uint32).view(np.float32)
