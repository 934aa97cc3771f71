"""Pins of the oracle's block encoders (qN_0 / qN_1) and bit packing.

* hand-derived worked examples (tests/golden/block_worked_examples.txt);
* round-trip error bounds that follow from the scale rule;
* code optimality by brute force over every level;
* special cases: zero block, constant block, sign flip, power-of-two scaling;
* packing against numpy.packbits (little-endian bit order) and an unpack round trip.
"""
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_worked_examples.txt")
NS = (2, 3, 4, 5, 6, 8)


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fmt, rule, d, m, hexbytes = line.split()
        rows.append((fmt, rule, int(d, 16), None if m == "-" else int(m, 16), bytes.fromhex(hexbytes)))
    return rows


@pytest.mark.parametrize("row", _golden(), ids=lambda r: r[0])
def test_worked_examples(row):
    fmt, rule, d_ref, m_ref, bytes_ref = row
    N = int(fmt[1])
    i = np.arange(32, dtype=np.float32)
    x = i - 16 if rule == "i-16" else i
    u = np.zeros(128, np.uint8)
    if fmt.endswith("_0"):
        d, u[:32] = O.encode_block_q0(N, x)
    else:
        d, m, u[:32] = O.encode_block_q1(N, x)
        assert m == m_ref
    assert d == d_ref
    assert O.pack_codes(N, u)[: 4 * N].tobytes() == bytes_ref


def _f16(h):
    return O.f64_from_fp16(h)


def _blocks(rng, n=200):
    out = []
    for k in range(n):
        scale = 10.0 ** rng.uniform(-3, 3)
        x = (rng.standard_normal(32) * scale).astype(np.float32)
        if k % 5 == 0:
            x[rng.integers(32)] *= 20           # an outlier
        if k % 7 == 0:
            x = np.abs(x)                       # one-signed block
        out.append(x)
    return out


@pytest.mark.parametrize("N", NS)
def test_q0_roundtrip_bound_and_optimality(N):
    rng = np.random.default_rng(100 + N)
    off = 1 << (N - 1)
    top = (1 << N) - 1
    for x in _blocks(rng):
        d, u = O.encode_block_q0(N, x)
        df = _f16(d)
        m = x[np.argmax(np.abs(x))]
        if x.max() == -x.min():
            m = x.max()
        # the scale is the fp16 rounding of m / -2^(N-1)
        assert abs(df - m / -off) <= abs(m / off) * 2.0**-11 + 2.0**-25
        xh = (u.astype(np.float64) - off) * df
        t = x.astype(np.float64) / df
        for i in range(32):
            if u[i] in (0, top):
                continue
            # non-clamped codes: the nearest level (brute force over all levels)
            lv = np.arange(top + 1) - off
            dist = np.abs(t[i] - lv)
            best = dist.min()
            assert dist[u[i]] <= best + 1e-6 * max(1.0, abs(t[i]))
            assert abs(x[i] - xh[i]) <= abs(df) * (0.5 + 1e-6)
        # clamped top code: at most one step
        assert np.all(np.abs(x - xh) <= abs(df) * (1.0 + 1e-6) + abs(m) * 2.0**-10)
        # the extreme element m reconstructs to -2^(N-1) * df
        im = int(np.argmax(np.abs(x))) if x.max() != -x.min() else int(np.argmax(x))
        assert u[im] == 0


@pytest.mark.parametrize("N", NS)
def test_q1_roundtrip_bound(N):
    rng = np.random.default_rng(200 + N)
    top = (1 << N) - 1
    for x in _blocks(rng):
        d, m, u = O.encode_block_q1(N, x)
        df, mf = _f16(d), _f16(m)
        mn, mx = float(x.min()), float(x.max())
        dq = (mx - mn) / top
        xh = mf + u.astype(np.float64) * df
        bound = df / 2 + abs(mf - mn) + top * abs(df - dq) + 4 * np.spacing(np.float32(max(abs(mn), abs(mx))))
        assert np.all(np.abs(x - xh) <= bound + 1e-12)
        # code optimality: nearest level of (x - mf)/df, brute force
        t = (x.astype(np.float64) - mf) / df
        for i in range(32):
            if 0 < u[i] < top:
                lv = np.arange(top + 1)
                dist = np.abs(t[i] - lv)
                assert dist[u[i]] <= dist.min() + 1e-6 * max(1.0, abs(t[i]))


@pytest.mark.parametrize("N", NS)
def test_special_cases(N):
    off = 1 << (N - 1)
    # all-zero block
    d, u = O.encode_block_q0(N, np.zeros(32, np.float32))
    assert d == 0 and np.all(u == off)
    d, m, u = O.encode_block_q1(N, np.zeros(32, np.float32))
    assert d == 0 and m == 0 and np.all(u == 0)
    # constant block, affine format: zero step, min = the constant
    d, m, u = O.encode_block_q1(N, np.full(32, 1.5, np.float32))
    assert d == 0 and m == O.fp16s_from_f32(1.5) and np.all(u == 0)
    rng = np.random.default_rng(300 + N)
    x = rng.standard_normal(32).astype(np.float32)
    # sign flip: identical codes, negated scale (needs a unique max-magnitude element)
    d1, u1 = O.encode_block_q0(N, x)
    d2, u2 = O.encode_block_q0(N, -x)
    assert np.array_equal(u1, u2) and d2 == (d1 ^ 0x8000)
    # power-of-two scaling in the normal fp16 range: identical codes, scale * 2^k
    for k in (-3, 1, 4):
        d3, u3 = O.encode_block_q0(N, (x * np.float32(2.0**k)).astype(np.float32))
        assert np.array_equal(u1, u3) and _f16(d3) == _f16(d1) * 2.0**k


def test_tie_goes_to_positive():
    x = np.zeros(32, np.float32)
    x[3], x[9] = 4.0, -4.0
    d, u = O.encode_block_q0(4, x)
    assert _f16(d) == -0.5 and u[3] == 0 and u[9] == 15


@pytest.mark.parametrize("N", NS)
def test_pack_against_numpy_packbits(N):
    rng = np.random.default_rng(400 + N)
    for _ in range(20):
        u = rng.integers(0, 1 << N, size=128).astype(np.uint8)
        bits = ((u[:, None] >> np.arange(N)[None, :]) & 1).astype(np.uint8).reshape(-1)
        ref = np.packbits(bits, bitorder="little")
        got = O.pack_codes(N, u)
        assert got.tobytes() == ref.tobytes()
        assert np.array_equal(O.unpack_codes(N, got), u)
        # block b occupies bytes [4N b, 4N (b+1))
        for b in range(4):
            ub = np.zeros(128, np.uint8)
            ub[32 * b: 32 * (b + 1)] = u[32 * b: 32 * (b + 1)]
            pb = O.pack_codes(N, ub)
            assert np.all(pb[: 4 * N * b] == 0) and np.all(pb[4 * N * (b + 1):] == 0)


def test_format_table():
    sizes = {"q2_0": 40, "q2_1": 48, "q3_0": 56, "q3_1": 64, "q4_0": 72, "q4_1": 80,
             "q5_0": 88, "q5_1": 96, "q6_0": 104, "q6_1": 112, "q8_0": 136, "q8_1": 144,
             "kvarn2": 42, "kvarn3": 58, "kvarn4": 74, "kvarn5": 90, "kvarn6": 106,
             "kvarn8": 138, "bf16": 256, "kvarn2_1": 50, "kvarn3_1": 66, "kvarn4_1": 82,
             "kvarn5_1": 98, "kvarn6_1": 114, "kvarn8_1": 146}
    for f, name in enumerate(O.FORMAT_NAMES):
        N, kind, cb, sb, pb = O.format_info(f)
        assert cb + sb + pb // 128 == sizes[name], name


@pytest.mark.parametrize("fmt", [f for f in range(1, 13)])
def test_token_dequant_roundtrip(fmt):
    """dequant(encode(x)) stays within one quantization step of x for every element."""
    rng = np.random.default_rng(500 + fmt)
    N, kind, cb, sb, pb = O.format_info(fmt)
    for _ in range(20):
        x = O.canon_bf16((rng.standard_normal(128) * 2).astype(np.float32))
        xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        codes, scales = O.encode_token(fmt, x)
        xh = O.dequant_token(fmt, codes, scales)
        for b in range(4):
            sl = slice(32 * b, 32 * (b + 1))
            if kind == O.KIND_Q0:
                step = abs(O.f64_from_fp16(int(scales[b])))
                assert np.all(np.abs(xf[sl] - xh[sl]) <= step * (1 + 1e-6))
            else:
                step = O.f64_from_fp16(int(scales[2 * b]))
                mf = O.f64_from_fp16(int(scales[2 * b + 1]))
                slack = abs(mf - xf[sl].min()) + ((1 << N) - 1) * abs(step - (xf[sl].max() - xf[sl].min()) / ((1 << N) - 1))
                assert np.all(np.abs(xf[sl] - xh[sl]) <= step / 2 + slack + 1e-6)


def test_bf16_identity_format():
    rng = np.random.default_rng(9)
    x = O.canon_bf16(rng.standard_normal(128).astype(np.float32))
    codes, scales = O.encode_token(O.BF16, x)
    assert codes.tobytes() == x.tobytes()
    assert np.array_equal(O.dequant_token(O.BF16, codes), (x.astype(np.uint32) << 16).view(np.float32))
