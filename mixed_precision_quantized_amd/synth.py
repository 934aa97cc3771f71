"""Seeded synthetic K/V/q generators shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the cache method itself: it only produces input
tensors.  It is the one piece of code both the HIP path and the CPU oracle are fed
from, so that they see bit-identical inputs.

Generator (counter-based, so any slice can be regenerated on its own, on the CPU or on
the GPU, with identical bits):
  * a 64-bit key per (workload seed, sequence, layer, KV head, stream) from the
    splitmix64 finalizer applied to a running combination of the ids;
  * element i of a stream (i = token*128 + dim) draws z = splitmix64(key + i*phi), where
    phi = 0x9E3779B97F4A7C15 and splitmix64 is Steele, Lea and Flood's SplitMix64
    output function;
  * the top 16 bits of z index a table of 65,536 quantiles of the target law at the
    midpoints (i+0.5)/65536: the standard normal, or Student's t with 3 degrees of
    freedom for heavy-tailed keys.  Table values are float32.
Outlier channels of K are picked per (layer, KV head) by a seeded Fisher-Yates shuffle
and multiplied (in float32) by a fixed factor.  Values are returned as float32; the
caller converts to bf16 with torch (round to nearest even) where the workload is bf16.

The integer hash runs on int64 tensors with two's-complement wrap-around, which torch
implements the same way on the CPU and on the GPU.
"""
from __future__ import annotations

import functools
import math

import numpy as np
import torch

MASK64 = (1 << 64) - 1
PHI = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
D = 128


def _s64(v: int) -> int:
    """Python int in [0, 2^64) -> the signed int64 with the same bits."""
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def splitmix64(x: int) -> int:
    """SplitMix64 output function on a Python integer (mod 2^64)."""
    z = (x + PHI) & MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def key(*ids: int) -> int:
    """Fold a tuple of non-negative ids into one 64-bit stream key."""
    k = 0x243F6A8885A308D3
    for i in ids:
        k = splitmix64(k ^ ((int(i) + 1) * PHI & MASK64))
    return k


def _lshr(z: torch.Tensor, s: int) -> torch.Tensor:
    return (z >> s) & ((1 << (64 - s)) - 1)


def hash_counters(k: int, start: int, n: int, device) -> torch.Tensor:
    """z_i = splitmix64(k + (start+i)*phi) for i < n, as int64 tensor bits."""
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    z = idx * _s64(PHI) + _s64(k + PHI)          # k + PHI + i*PHI  (mod 2^64)
    z = (z ^ _lshr(z, 30)) * _s64(M1)
    z = (z ^ _lshr(z, 27)) * _s64(M2)
    z = z ^ _lshr(z, 31)
    return z


@functools.lru_cache(maxsize=None)
def _table_np(law: str) -> np.ndarray:
    from scipy import special
    p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    if law == "normal":
        v = special.ndtri(p)
    elif law == "t3":
        v = special.stdtrit(3, p)
    else:
        raise ValueError(law)
    return v.astype(np.float32)


_TABLES: dict = {}


def _table(law: str, device) -> torch.Tensor:
    dkey = (law, str(device))
    t = _TABLES.get(dkey)
    if t is None:
        t = torch.from_numpy(_table_np(law)).to(device)
        _TABLES[dkey] = t
    return t


def draw(k: int, start: int, n: int, law: str = "normal", device="cpu") -> torch.Tensor:
    """n float32 draws of the given law for counters start..start+n-1 of stream k."""
    z = hash_counters(k, start, n, device)
    idx = _lshr(z, 48)
    return _table(law, device)[idx]


def pick_channels(k: int, count: int, d: int = D) -> list:
    """Seeded Fisher-Yates shuffle of range(d); the first `count` entries."""
    perm = list(range(d))
    state = k
    for i in range(d - 1, 0, -1):
        state = splitmix64(state)
        j = state % (i + 1)
        perm[i], perm[j] = perm[j], perm[i]
    return sorted(perm[:count])


# ------------------------------------------------------------------ workload recipes
# Seeds are 0x4B560000 + workload index.  Shapes follow the workloads the pages discuss:
# 64 layers x 8 KV heads x head_dim 128 at 240k tokens (the arithmetic example of the
# first page), and 64k-context sweeps (the KLD table of the release post).
WORKLOADS = {
    "c1_q4_0_ctx4096": dict(index=0, layers=1, kv_heads=1, q_heads=4, ctx=4096, tail=256,
                           fmts=("q4_0",), in_dtype="f32", k_law="normal",
                           outliers=2, outlier_mult=20.0),
    "c2_sweep_ctx65536": dict(index=1, layers=1, kv_heads=8, q_heads=32, ctx=65536,
                              tails=(0, 1024, 2048),
                              fmts=("q2_0", "q2_1", "q3_0", "q3_1", "q4_0", "q5_0", "q6_0",
                                    "q6_1", "q8_0"),
                              in_dtype="bf16", k_law="normal", outliers=4, outlier_mult=15.0),
    "c3_kvarn_ctx65536": dict(index=2, layers=1, kv_heads=8, q_heads=32, ctx=65536, tail=1024,
                              fmts=("kvarn2", "kvarn3", "kvarn4"), in_dtype="bf16",
                              k_law="t3", outliers=4, outlier_mult=15.0),
    "c4_ctx240000_64l": dict(index=3, layers=64, kv_heads=8, q_heads=32, ctx=240000, tail=2048,
                             fmts=("kvarn4", "q4_0"), in_dtype="bf16", k_law="normal",
                             outliers=4, outlier_mult=15.0),
    "c5_ragged16_64l": dict(index=4, layers=64, kv_heads=8, q_heads=32, n_seqs=16,
                            len_lo=8000, len_hi=120000, tail=1024, chunk=512,
                            fmts=("kvarn3",), in_dtype="bf16", k_law="normal",
                            outliers=4, outlier_mult=15.0),
}


def seed_of(workload: str) -> int:
    return 0x4B560000 + WORKLOADS[workload]["index"]


def kv_rows(workload: str, seq: int, layer: int, head: int, is_v: int, t0: int, t1: int,
            device="cpu") -> torch.Tensor:
    """float32 [t1-t0][128] values of one stream for tokens t0..t1-1."""
    w = WORKLOADS[workload]
    s = seed_of(workload)
    k = key(s, seq, layer, head, is_v)
    law = w["k_law"] if not is_v else "normal"
    x = draw(k, t0 * D, (t1 - t0) * D, law, device).view(t1 - t0, D)
    if not is_v and w.get("outliers", 0):
        ch = pick_channels(key(s, 0xC4A7, layer, head), w["outliers"])
        mult = torch.ones(D, dtype=torch.float32, device=device)
        mult[ch] = float(w["outlier_mult"])
        x = x * mult
    return x


def q_rows(workload: str, seq: int, layer: int, step: int, q_heads: int, device="cpu"):
    """float32 [q_heads][128] query of one sequence at one decode step."""
    k = key(seed_of(workload), 0x9999, seq, layer, step)
    return draw(k, 0, q_heads * D, "normal", device).view(q_heads, D)


def seq_lengths(workload: str) -> list:
    """Ragged lengths, uniform on the integers [len_lo, len_hi]."""
    w = WORKLOADS[workload]
    st = key(seed_of(workload), 0x1E9)
    out = []
    span = w["len_hi"] - w["len_lo"] + 1
    for _ in range(w["n_seqs"]):
        st = splitmix64(st)
        out.append(w["len_lo"] + st % span)
    return out


def to_bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """float32 tensor -> bf16 tensor (torch's round to nearest even)."""
    return x.to(torch.bfloat16)


def bf16_as_u16(x: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def softmax_scale() -> float:
    return 1.0 / math.sqrt(D)
