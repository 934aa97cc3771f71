"""The KVarN pins catch plausible mistakes: each case below plants one mistake in a copy of
the oracle's C source (on the CPU, in a temporary directory), builds it with the oracle's
own flags and runs the hand-derived checks of test_oracle_kvarn_pins against it.  Every
mutant must fail at least one check, and the unmodified copy must pass them all.

Planted mistakes: the Sinkhorn sums taken sequentially (either direction) or as an
adjacent-pair tree instead of the halving tree; a division in place of the reciprocal
product (row or column step); the channel-scale guard dropped or set to another value.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle as O
from oracle import build as oracle_build

import test_oracle_kvarn_pins as P

_f32p = ctypes.POINTER(ctypes.c_float)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)

TREE = ("    for (int w = 64; w >= 1; w >>= 1)\n"
        "        for (int i = 0; i < w; ++i) v[i] = v[i] + v[i + w];\n"
        "    return v[0];")

MUTANTS = {
    "sequential_sum": (TREE, "    float s = 0.0f;\n    for (int i = 0; i < 128; ++i) s = s + v[i];\n    return s;"),
    "reverse_sequential_sum": (TREE, "    float s = 0.0f;\n    for (int i = 127; i >= 0; --i) s = s + v[i];\n    return s;"),
    "adjacent_pair_tree": (TREE, "    for (int w = 1; w < 128; w <<= 1)\n"
                                 "        for (int i = 0; i + w < 128; i += 2 * w) v[i] = v[i] + v[i + w];\n"
                                 "    return v[0];"),
    "row_step_division": ("v[j] = A[t * 128 + j] * ic[j];", "v[j] = A[t * 128 + j] / c2[j];"),
    "column_step_division": ("v[t] = A[t * 128 + j] * ir[t];", "v[t] = A[t * 128 + j] / r2[t];"),
    "no_channel_guard": ("if (c == 0) c = 0x3C00u;", ";"),
    "channel_guard_half": ("if (c == 0) c = 0x3C00u;", "if (c == 0) c = 0x3800u;"),
}


def _build(tmp, name, src_text):
    src = os.path.join(tmp, name + ".c")
    with open(src, "w") as f:
        f.write(src_text)
    lib = os.path.join(tmp, "lib" + name + ".so")
    inc = os.path.dirname(oracle_build.SRC)
    subprocess.run(["gcc"] + oracle_build.CFLAGS + ["-I" + inc, "-o", lib, src, "-lm"], check=True)
    L = ctypes.CDLL(lib)
    L.kvo_sinkhorn128.argtypes = [_f32p, ctypes.c_int, _f32p, _f32p]
    L.kvo_sinkhorn128.restype = None
    L.kvo_encode_page_kvarn.argtypes = [ctypes.c_int, _u16p, _u8p, _u16p, _u16p]
    L.kvo_encode_page_kvarn.restype = None

    def sinkhorn(A, iters):
        A = np.ascontiguousarray(A, dtype=np.float32)
        r2 = np.zeros(128, np.float32)
        c2 = np.zeros(128, np.float32)
        L.kvo_sinkhorn128(A.ctypes.data_as(_f32p), iters, r2.ctypes.data_as(_f32p), c2.ctypes.data_as(_f32p))
        return r2, c2

    def encode_page(N, X):
        X = np.ascontiguousarray(X, dtype=np.uint16)
        codes = np.zeros((128, 16 * N), np.uint8)
        scales = np.zeros((128, 4), np.uint16)
        cscale = np.zeros(128, np.uint16)
        with np.errstate(all="ignore"):
            L.kvo_encode_page_kvarn(N, X.ctypes.data_as(_u16p), codes.ctypes.data_as(_u8p),
                                    scales.ctypes.data_as(_u16p), cscale.ctypes.data_as(_u16p))
        return codes, scales, cscale

    return sinkhorn, encode_page


def _failures(sinkhorn, encode_page):
    failed = []
    for name, fn in (("order", lambda: P.check_sinkhorn_order(sinkhorn)),
                     ("guard", lambda: P.check_guard_page(encode_page, 4))):
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def _source():
    with open(oracle_build.SRC) as f:
        return f.read()


def test_unmodified_copy_passes(tmp_path):
    s, e = _build(str(tmp_path), "control", _source())
    assert _failures(s, e) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = _source()
    assert text.count(old) == 1, "mutation site of %s not found exactly once in the oracle" % name
    s, e = _build(str(tmp_path), name, text.replace(old, new))
    assert _failures(s, e), "the pins did not catch the planted mistake %s" % name
