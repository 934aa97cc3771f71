"""ctypes view of the CPU oracle (oracle/kvq_oracle.c).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import this package.  The HIP library never does, and shares no code
with it.  All arrays cross the boundary as contiguous numpy arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

# Format numbering (an interface value shared with the library header, same integers).
BF16, Q2_0, Q2_1, Q3_0, Q3_1, Q4_0, Q4_1, Q5_0, Q5_1, Q6_0, Q6_1, Q8_0, Q8_1, \
    KVARN2, KVARN3, KVARN4, KVARN5, KVARN6, KVARN8, \
    KVARN2_1, KVARN3_1, KVARN4_1, KVARN5_1, KVARN6_1, KVARN8_1 = range(25)
FORMAT_NAMES = ["bf16", "q2_0", "q2_1", "q3_0", "q3_1", "q4_0", "q4_1", "q5_0", "q5_1",
                "q6_0", "q6_1", "q8_0", "q8_1", "kvarn2", "kvarn3", "kvarn4", "kvarn5",
                "kvarn6", "kvarn8", "kvarn2_1", "kvarn3_1", "kvarn4_1", "kvarn5_1", "kvarn6_1",
                "kvarn8_1"]
KIND_BF16, KIND_Q0, KIND_Q1, KIND_KVARN, KIND_KVARN1 = range(5)

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int)


def lib():
    """Load (building first if absent) the oracle library."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.kvo_bf16_from_f32.argtypes = [ctypes.c_float]
        L.kvo_bf16_from_f32.restype = ctypes.c_uint16
        L.kvo_f32_from_bf16.argtypes = [ctypes.c_uint16]
        L.kvo_f32_from_bf16.restype = ctypes.c_float
        L.kvo_fp16s_from_f32.argtypes = [ctypes.c_float]
        L.kvo_fp16s_from_f32.restype = ctypes.c_uint16
        L.kvo_f64_from_fp16.argtypes = [ctypes.c_uint16]
        L.kvo_f64_from_fp16.restype = ctypes.c_double
        L.kvo_format_info.argtypes = [ctypes.c_int] + [_i32p] * 5
        L.kvo_format_info.restype = ctypes.c_int
        L.kvo_encode_block_q0.argtypes = [ctypes.c_int, _f32p, _u16p, _u8p]
        L.kvo_encode_block_q0.restype = None
        L.kvo_encode_block_q1.argtypes = [ctypes.c_int, _f32p, _u16p, _u16p, _u8p]
        L.kvo_encode_block_q1.restype = None
        L.kvo_pack_codes.argtypes = [ctypes.c_int, _u8p, _u8p]
        L.kvo_pack_codes.restype = None
        L.kvo_unpack_codes.argtypes = [ctypes.c_int, _u8p, _u8p]
        L.kvo_unpack_codes.restype = None
        L.kvo_fwht128_f32.argtypes = [_f32p]
        L.kvo_fwht128_f32.restype = None
        L.kvo_sinkhorn128.argtypes = [_f32p, ctypes.c_int, _f32p, _f32p]
        L.kvo_sinkhorn128.restype = None
        L.kvo_encode_page_kvarn.argtypes = [ctypes.c_int, _u16p, _u8p, _u16p, _u16p]
        L.kvo_encode_page_kvarn.restype = None
        L.kvo_encode_page_kvarn_q1.argtypes = [ctypes.c_int, _u16p, _u8p, _u16p, _u16p]
        L.kvo_encode_page_kvarn_q1.restype = None
        L.kvo_encode_token.argtypes = [ctypes.c_int, _u16p, _u8p, _u16p]
        L.kvo_encode_token.restype = ctypes.c_int
        L.kvo_encode_stream.argtypes = [ctypes.c_int, ctypes.c_int64, _u16p, _u8p, _u16p, _u16p]
        L.kvo_encode_stream.restype = ctypes.c_int
        L.kvo_dequant_token.argtypes = [ctypes.c_int, _u8p, _u16p, _u16p, _f64p]
        L.kvo_dequant_token.restype = ctypes.c_int
        L.kvo_dequant_stream.argtypes = [ctypes.c_int, ctypes.c_int64, _u8p, _u16p, _u16p, _f64p]
        L.kvo_dequant_stream.restype = ctypes.c_int
        L.kvo_granule.argtypes = [ctypes.c_int, ctypes.c_int]
        L.kvo_granule.restype = ctypes.c_int64
        L.kvo_ring_capacity.argtypes = [ctypes.c_int64, ctypes.c_int64]
        L.kvo_ring_capacity.restype = ctypes.c_int64
        L.kvo_nq_after.argtypes = [ctypes.c_int64] * 4
        L.kvo_nq_after.restype = ctypes.c_int64
        L.kvo_ring_image.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _u16p, _u16p]
        L.kvo_ring_image.restype = ctypes.c_int
        L.kvo_attention.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    _u8p, _u16p, _u16p, _u8p, _u16p, _u16p, _u16p, _u16p,
                                    ctypes.c_int, _f64p, ctypes.c_double, _f64p]
        L.kvo_attention.restype = ctypes.c_int
        L.kvo_set_canonical_f16.argtypes = [ctypes.c_int]
        L.kvo_set_canonical_f16.restype = None
        L.kvo_canonical_f16.argtypes = []
        L.kvo_canonical_f16.restype = ctypes.c_int
        L.kvo_prefill_attention.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                            ctypes.c_int, _u8p, _u16p, _u16p, _u8p, _u16p, _u16p, _u16p,
                                            _u16p, ctypes.c_int, _f64p, ctypes.c_double, _f64p]
        L.kvo_prefill_attention.restype = ctypes.c_int
        L.kvo_attention_kld.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, _u8p, _u16p, _u16p,
                                        _u16p, ctypes.c_int, _f64p, ctypes.c_double, _f64p]
        L.kvo_attention_kld.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _p(a, t):
    if a is None:
        return ctypes.cast(None, t)
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


# ---------------------------------------------------------------- scalar helpers
def bf16_from_f32(x: float) -> int:
    return int(lib().kvo_bf16_from_f32(float(x)))


def f32_from_bf16(b: int) -> float:
    return float(lib().kvo_f32_from_bf16(int(b)))


def fp16s_from_f32(x: float) -> int:
    return int(lib().kvo_fp16s_from_f32(float(x)))


def f64_from_fp16(h: int) -> float:
    return float(lib().kvo_f64_from_fp16(int(h)))


def set_canonical_f16(on: bool) -> None:
    """Canonical 16-bit type of the values the oracle encodes and attends over: bf16
    (default) or binary16 (an F16 tail).  Process-wide; see canonical()."""
    lib().kvo_set_canonical_f16(1 if on else 0)


def canonical_f16() -> bool:
    return bool(lib().kvo_canonical_f16())


class canonical:
    """with canonical("f16"): ... -- the oracle's canonical type inside the block."""

    def __init__(self, dtype: str):
        assert dtype in ("bf16", "f16")
        self.on = dtype == "f16"

    def __enter__(self):
        self.prev = canonical_f16()
        set_canonical_f16(self.on)
        return self

    def __exit__(self, *exc):
        set_canonical_f16(self.prev)
        return False


def canon_f16(x: np.ndarray) -> np.ndarray:
    """Canonical binary16 bits of token values: float32 values, or bf16 bits (uint16), to
    the nearest binary16 (ties to even), saturated to +-65504, zero as +0 -- the oracle's
    scalar kvo_fp16s_from_f32, vectorized (numpy's float16 cast rounds to nearest even)."""
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << 16).view(np.float32)
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.clip(x, -65504.0, 65504.0).astype(np.float16)
    y[y == 0] = 0.0
    return y.view(np.uint16)


def canon(x: np.ndarray) -> np.ndarray:
    """Canonical 16-bit bits of token values in the current canonical type."""
    return canon_f16(x) if canonical_f16() else canon_bf16(x)


def canon_bf16(x: np.ndarray) -> np.ndarray:
    """Canonical token values: fp32 -> bf16 bits (round to nearest even), elementwise
    through the oracle's scalar conversion; bf16 (uint16) input passes unchanged."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x)
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = lib().kvo_bf16_from_f32
    out = np.empty(x.shape, np.uint16)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = f(float(flat_in[i]))
    return out


def format_info(fmt: int):
    """(bits, kind, code_bytes, scale_bytes, page_bytes) of a format."""
    vals = [ctypes.c_int() for _ in range(5)]
    rc = lib().kvo_format_info(fmt, *[ctypes.byref(v) for v in vals])
    if rc != 0:
        raise ValueError("bad format %r" % fmt)
    return tuple(v.value for v in vals)


# ---------------------------------------------------------------- block / token
def encode_block_q0(N: int, x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape == (32,)
    d = ctypes.c_uint16()
    u = np.zeros(32, np.uint8)
    lib().kvo_encode_block_q0(N, _p(x, _f32p), ctypes.byref(d), _p(u, _u8p))
    return int(d.value), u


def encode_block_q1(N: int, x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape == (32,)
    d = ctypes.c_uint16()
    m = ctypes.c_uint16()
    u = np.zeros(32, np.uint8)
    lib().kvo_encode_block_q1(N, _p(x, _f32p), ctypes.byref(d), ctypes.byref(m), _p(u, _u8p))
    return int(d.value), int(m.value), u


def pack_codes(N: int, u) -> np.ndarray:
    u = np.ascontiguousarray(u, dtype=np.uint8)
    assert u.shape == (128,)
    out = np.zeros(16 * N, np.uint8)
    lib().kvo_pack_codes(N, _p(u, _u8p), _p(out, _u8p))
    return out


def unpack_codes(N: int, b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    assert b.shape == (16 * N,)
    out = np.zeros(128, np.uint8)
    lib().kvo_unpack_codes(N, _p(b, _u8p), _p(out, _u8p))
    return out


def fwht128(y) -> np.ndarray:
    y = np.array(y, dtype=np.float32, copy=True)
    assert y.shape == (128,)
    lib().kvo_fwht128_f32(_p(y, _f32p))
    return y


def sinkhorn128(A, iters: int = 8):
    A = np.ascontiguousarray(A, dtype=np.float32)
    assert A.shape == (128, 128)
    r2 = np.zeros(128, np.float32)
    c2 = np.zeros(128, np.float32)
    lib().kvo_sinkhorn128(_p(A, _f32p), iters, _p(r2, _f32p), _p(c2, _f32p))
    return r2, c2


def encode_page_kvarn(N: int, X_bf16, affine: bool = False):
    """One KVarN page; affine: the qN_1 inner quantizer (scales [128][4][2] {d, m})."""
    X = np.ascontiguousarray(X_bf16, dtype=np.uint16)
    assert X.shape == (128, 128)
    codes = np.zeros((128, 16 * N), np.uint8)
    scales = np.zeros((128, 8) if affine else (128, 4), np.uint16)
    cscale = np.zeros(128, np.uint16)
    f = lib().kvo_encode_page_kvarn_q1 if affine else lib().kvo_encode_page_kvarn
    f(N, _p(X, _u16p), _p(codes, _u8p), _p(scales, _u16p), _p(cscale, _u16p))
    return codes, scales, cscale


def encode_token(fmt: int, x_bf16):
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    N, kind, cb, sb, pb = format_info(fmt)
    codes = np.zeros(cb, np.uint8)
    scales = np.zeros(max(sb // 2, 1), np.uint16)
    rc = lib().kvo_encode_token(fmt, _p(x, _u16p), _p(codes, _u8p), _p(scales, _u16p))
    if rc != 0:
        raise ValueError("encode_token rc=%d" % rc)
    return codes, scales[: sb // 2]


def encode_stream(fmt: int, n_q: int, x_bf16):
    """Encode rows [0, n_q) of one stream; returns (codes, scales, cscale)."""
    x = np.ascontiguousarray(x_bf16[:n_q], dtype=np.uint16)
    N, kind, cb, sb, pb = format_info(fmt)
    codes = np.zeros((n_q, cb), np.uint8)
    scales = np.zeros((n_q, max(sb // 2, 1)), np.uint16)
    cscale = np.zeros((max(n_q // 128, 1), 128), np.uint16)
    rc = lib().kvo_encode_stream(fmt, n_q, _p(x, _u16p), _p(codes, _u8p), _p(scales, _u16p),
                                 _p(cscale, _u16p))
    if rc != 0:
        raise ValueError("encode_stream rc=%d" % rc)
    return codes, scales[:, : sb // 2], cscale[: n_q // 128] if kind in (KIND_KVARN, KIND_KVARN1) else None


def dequant_token(fmt: int, codes, scales=None, cscale_row=None) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    sc = None if scales is None else np.ascontiguousarray(scales, dtype=np.uint16)
    cr = None if cscale_row is None else np.ascontiguousarray(cscale_row, dtype=np.uint16)
    out = np.zeros(128, np.float64)
    rc = lib().kvo_dequant_token(fmt, _p(codes, _u8p), _p(sc, _u16p), _p(cr, _u16p),
                                 _p(out, _f64p))
    if rc != 0:
        raise ValueError("dequant_token rc=%d" % rc)
    return out


def dequant_stream(fmt: int, n_q: int, codes, scales, cscale) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    sc = None if scales is None or scales.size == 0 else np.ascontiguousarray(scales, dtype=np.uint16)
    cs = None if cscale is None else np.ascontiguousarray(cscale, dtype=np.uint16)
    out = np.zeros((n_q, 128), np.float64)
    rc = lib().kvo_dequant_stream(fmt, n_q, _p(codes, _u8p), _p(sc, _u16p), _p(cs, _u16p),
                                  _p(out, _f64p))
    if rc != 0:
        raise ValueError("dequant_stream rc=%d" % rc)
    return out


# ---------------------------------------------------------------- state machine
def granule(fmt_k: int, fmt_v: int) -> int:
    return int(lib().kvo_granule(fmt_k, fmt_v))


def ring_capacity(T: int, G: int) -> int:
    return int(lib().kvo_ring_capacity(T, G))


def nq_after(n_q: int, n: int, keep: int, G: int) -> int:
    return int(lib().kvo_nq_after(n_q, n, keep, G))


def ring_image(n: int, n_q: int, R: int, x_bf16, ring=None) -> np.ndarray:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    if ring is None:
        ring = np.zeros((max(R, 1), 128), np.uint16)
    rc = lib().kvo_ring_image(n, n_q, R, _p(x, _u16p), _p(ring, _u16p))
    if rc != 0:
        raise ValueError("ring_image rc=%d" % rc)
    return ring


# ---------------------------------------------------------------- attention
def attention(n, n_q, fmt_k, fmt_v, kq, vq, k_tail, v_tail, q, sigma):
    """kq/vq: (codes, scales, cscale) tuples of rows [0, n_q); k_tail/v_tail: bf16 rows of
    tokens [n_q, n) in token order; q: [g][128] float values.  Returns [g][128] float64."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    g = q.shape[0]
    out = np.zeros((g, 128), np.float64)

    def parts(t):
        c, s, cs = t
        c = np.ascontiguousarray(c, dtype=np.uint8) if c is not None and c.size else None
        s = np.ascontiguousarray(s, dtype=np.uint16) if s is not None and s.size else None
        cs = np.ascontiguousarray(cs, dtype=np.uint16) if cs is not None and cs.size else None
        return _p(c, _u8p), _p(s, _u16p), _p(cs, _u16p)

    kt = np.ascontiguousarray(k_tail, dtype=np.uint16) if n > n_q else None
    vt = np.ascontiguousarray(v_tail, dtype=np.uint16) if n > n_q else None
    rc = lib().kvo_attention(int(n), int(n_q), fmt_k, fmt_v, *parts(kq), *parts(vq),
                             _p(kt, _u16p), _p(vt, _u16p), g, _p(q, _f64p), float(sigma),
                             _p(out, _f64p))
    if rc != 0:
        raise ValueError("attention rc=%d" % rc)
    return out


def attention_kld(n, n_q, fmt_k, kq, k_exact, q, sigma):
    """KL(P || Q) per query head: P over the exact bf16 keys k_exact ([n][128] bits, every
    token), Q over the cache's keys (kq = (codes, scales, cscale) of rows [0, n_q), the
    exact rows after).  q: [g][128] values.  Returns [g] float64."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    g = q.shape[0]
    out = np.zeros(g, np.float64)
    c, s, cs = kq if kq is not None else (None, None, None)
    c = np.ascontiguousarray(c, dtype=np.uint8) if c is not None and c.size else None
    s = np.ascontiguousarray(s, dtype=np.uint16) if s is not None and s.size else None
    cs = np.ascontiguousarray(cs, dtype=np.uint16) if cs is not None and cs.size else None
    ke = np.ascontiguousarray(k_exact, dtype=np.uint16)
    rc = lib().kvo_attention_kld(int(n), int(n_q), fmt_k, _p(c, _u8p), _p(s, _u16p), _p(cs, _u16p),
                                 _p(ke, _u16p), g, _p(q, _f64p), float(sigma), _p(out, _f64p))
    if rc != 0:
        raise ValueError("attention_kld rc=%d" % rc)
    return out


def prefill_attention(n, n_q, n_new, fmt_k, fmt_v, kq, vq, k_tail, v_tail, q, sigma):
    """Causal attention of the last n_new tokens: q [n_new][g][128] values; kq/vq as in
    attention(); k_tail/v_tail: bf16 rows of tokens [n_q, n).  Returns [n_new][g][128]."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    n_new_, g = q.shape[0], q.shape[1]
    assert n_new_ == n_new
    out = np.zeros((n_new, g, 128), np.float64)

    def parts(t):
        if t is None:
            return None, None, None
        c, s, cs = t
        c = np.ascontiguousarray(c, dtype=np.uint8) if c is not None and c.size else None
        s = np.ascontiguousarray(s, dtype=np.uint16) if s is not None and s.size else None
        cs = np.ascontiguousarray(cs, dtype=np.uint16) if cs is not None and cs.size else None
        return _p(c, _u8p), _p(s, _u16p), _p(cs, _u16p)

    kt = np.ascontiguousarray(k_tail, dtype=np.uint16) if n > n_q else None
    vt = np.ascontiguousarray(v_tail, dtype=np.uint16) if n > n_q else None
    rc = lib().kvo_prefill_attention(int(n), int(n_q), int(n_new), fmt_k, fmt_v, *parts(kq), *parts(vq),
                                     _p(kt, _u16p), _p(vt, _u16p), g, _p(q, _f64p), float(sigma),
                                     _p(out, _f64p))
    if rc != 0:
        raise ValueError("prefill_attention rc=%d" % rc)
    return out
