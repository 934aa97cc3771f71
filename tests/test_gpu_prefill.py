"""GPU parity of chunked-prefill attention (kv_prefill_attn) against the oracle's binary64
causal attention over the same cache, through the C ABI.

Small cases: a sequence of n tokens whose last n_new form the chunk (appended last, in
ragged pieces), for tails that keep the whole chunk in the BF16 ring, split it across the
boundary, or quantize it entirely; every query and every head compared, normwise per
(query, head) within 2e-3 (the decode bound: keys are used exactly, the query and the
probabilities are rounded to binary16 once, values are dequantized to binary16; a CPU
model of these roundings on the 64k KVarN workload gives <= 7e-4).  Full size: a 512-token
chunk at the end of a 65,536-token sequence, 8 KV heads, sampled queries checked against
the decode oracle (the chunk's queries all see the whole quantized region).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_quantized_amd import kvq

import kvq_testlib as T

pytestmark = pytest.mark.gpu
SIGMA = 1.0 / math.sqrt(128)
TOL = 2e-3


def _err(got, ref):
    g = got.reshape(-1, 128).astype(np.float64)
    r = ref.reshape(-1, 128)
    return float(np.max(np.abs(g - r).max(axis=1) / np.abs(r).max(axis=1)))


def _prefill_case(fmt, n, n_new, tail, H=2):
    wl = "c3_kvarn_ctx65536" if "kvarn" in fmt else "c2_sweep_ctx65536"
    cache = T.make_cache(fmt, 1, H, 4 * H, tail_tokens=tail, n_seqs=1, max_tokens=n)
    T.fill(cache, wl, 0, [0], H, n - n_new, T.chunk_list(n - n_new, [777, 1, 300]))
    T.fill(cache, wl, 0, [0], H, n_new, T.chunk_list(n_new, [max(1, n_new // 3), 1]), t_start=n - n_new)
    qs = torch.stack([T.query(wl, 0, 0, step, 4 * H, "cuda") for step in range(n_new)], 0).contiguous()
    out = cache.prefill(0, 0, qs).cpu().numpy()
    n_, n_q = cache.seq_get(0, 0)
    assert n_ == n
    qv = T.query_values(qs)
    fk, fv = (O.FORMAT_NAMES.index(x) for x in T.split_fmt(fmt))
    worst = 0.0
    for h in range(H):
        k = T.canon_rows(wl, 0, 0, h, 0, 0, n)
        v = T.canon_rows(wl, 0, 0, h, 1, 0, n)
        kq = O.encode_stream(fk, n_q, k) if n_q else None
        vq = O.encode_stream(fv, n_q, v) if n_q else None
        ref = O.prefill_attention(n, n_q, n_new, fk, fv, kq, vq, k[n_q:], v[n_q:], qv[:, 4 * h:4 * h + 4], SIGMA)
        e = _err(out[:, 4 * h:4 * h + 4], ref)
        assert e <= TOL, "%s tail %d head %d: rel err %.3g" % (fmt, tail, h, e)
        worst = max(worst, e)
    return worst


@pytest.mark.parametrize("tail", [0, 100, 1024])
@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "q3_1", "q2_0", "kvarn4", "kvarn2", "bf16", "q4_1/kvarn4",
                                 "kvarn3/q5_1", "kvarn4_1", "kvarn3_1/q4_1", "q4_0/kvarn2_1", "kvarn8_1/kvarn4"])
def test_prefill_matches_oracle(fmt, tail):
    _prefill_case(fmt, 1500, 160, tail)


def test_prefill_chunk_512_partial_tile():
    _prefill_case("kvarn4", 3000, 500, 1024)


# shapes at the edges of the launch plan: every token in the ring (no quantized split), no
# ring (no ring split), a one-token chunk (one tile, the other half of its pair empty), a
# chunk that is the whole sequence, and three tiles (an odd count) over several pages
@pytest.mark.parametrize("fmt,n,n_new,tail", [("kvarn4", 700, 160, 1024), ("q4_0", 700, 96, 0),
                                              ("kvarn3/q4_1", 1300, 1, 200), ("q8_0", 257, 257, 64),
                                              ("kvarn4_1", 900, 70, 0), ("bf16", 600, 33, 100)])
def test_prefill_plan_edges(fmt, n, n_new, tail):
    _prefill_case(fmt, n, n_new, tail)


def test_prefill_full_size_sampled():
    wl = "c3_kvarn_ctx65536"
    n, n_new, H = 65536, 512, 8
    cache = kvq.Cache(1, H, 32, "kvarn4", tail_tokens=1024, n_seqs=1, max_tokens=n)
    T.fill(cache, wl, 0, [0], H, n, [16384] * 4)
    qs = torch.stack([T.query(wl, 0, 0, step, 32, "cuda") for step in range(n_new)], 0).contiguous()
    out = cache.prefill(0, 0, qs).cpu().numpy()
    _, n_q = cache.seq_get(0, 0)
    qv = T.query_values(qs)
    f = O.KVARN4
    for h in (0, 5):
        k = T.canon_rows(wl, 0, 0, h, 0, 0, n)
        v = T.canon_rows(wl, 0, 0, h, 1, 0, n)
        kq, vq = O.encode_stream(f, n_q, k), O.encode_stream(f, n_q, v)
        for i in (0, 1, 255, 511):
            ctx = n - n_new + i + 1
            ref = O.attention(ctx, n_q, f, f, kq, vq, k[n_q:ctx], v[n_q:ctx], qv[i, 4 * h:4 * h + 4], SIGMA)
            e = _err(out[i, 4 * h:4 * h + 4], ref)
            assert e <= TOL, "query %d head %d: rel err %.3g" % (i, h, e)


def test_prefill_errors():
    cache = kvq.Cache(1, 1, 4, "q4_0", tail_tokens=0, n_seqs=1, max_tokens=256)
    q = torch.zeros(4, 4, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvq.KVError):
        cache.prefill(0, 0, q)                              # empty sequence
