"""GPU parity at the workloads' full sizes, through the C ABI, in the launch configuration of
the benchmark (same library entry points, same split planner).

  * 65,536-token sweep: every (format, tail) pair of the block-format sweep, the three
    KVarN formats and kvarn4_1, one layer x 8 KV heads x 32 query heads.  Codes, block scales, channel
    scales and live ring rows of all 16 streams byte-identical to the oracle; decode
    attention of all 32 query heads within 2e-3 (normwise per head) of the oracle's
    binary64 attention over the same dequantized values.
  * 240,000-token decode step: 64 layers x 8 KV heads, kvarn4 and q4_0, tail 2048; the
    same comparisons on sampled layers 0, 31 and 63 (all heads, both streams).
  * Ragged batch: 16 sequences of 8k-120k tokens, 64 layers, kvarn3, tail 1024, batched
    appends, one 512-token append step that spills the tail, batched decode before and
    after it; sampled (sequence, layer, head) units compared.

Oracle inputs come from the CPU side of the seeded generator; the device fills its cache
from the GPU side of the same generator (bit-identity of the two is checked separately).
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_quantized_amd import kvq, synth

import kvq_testlib as T

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
TOL = 2e-3
SIGMA = 1.0 / math.sqrt(128)
POOL = ThreadPoolExecutor(max(4, min(16, os.cpu_count() or 4)))


def _pmap(fn, items):
    return list(POOL.map(fn, items))


def _release():
    """Return freed device memory (the caller has dropped its cache) before the next test."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _check_units(cache, fmt, wl, units, rows, q_by_seq, out_by_seq, group=4):
    """Byte parity of both streams and attention of every (seq, layer, head) unit."""
    def streams(u):
        seq, layer, head = u
        for is_v in (0, 1):
            T.compare_stream(cache, fmt, rows[(seq, layer, head, is_v)], seq, layer, head, is_v)
        return u

    _pmap(streams, units)

    def attn(u):
        seq, layer, head = u
        n, n_q = cache.seq_get(seq, layer)
        qv = q_by_seq[(seq, layer)][head * group:(head + 1) * group]
        ref = T.oracle_attention(fmt, rows[(seq, layer, head, 0)], rows[(seq, layer, head, 1)], n, n_q, qv, SIGMA)
        got = out_by_seq[(seq, layer)][head * group:(head + 1) * group]
        return u, T.rel_err(got, ref)

    worst = 0.0
    for u, e in _pmap(attn, units):
        assert e <= TOL, "attention %s seq %d layer %d head %d: rel err %.3g" % ((fmt,) + u + (e,))
        worst = max(worst, e)
    return worst


# --------------------------------------------------------------------------------------
# 65,536-token sweeps (one layer, 8 KV heads, 32 query heads)

N64K = 65536


@pytest.fixture(scope="module")
def rows_c2():
    wl = "c2_sweep_ctx65536"
    keys = [(0, 0, h, v) for h in range(8) for v in (0, 1)]
    vals = _pmap(lambda k: T.canon_rows(wl, k[0], k[1], k[2], k[3], 0, N64K), keys)
    return dict(zip(keys, vals))


@pytest.fixture(scope="module")
def rows_c3():
    wl = "c3_kvarn_ctx65536"
    keys = [(0, 0, h, v) for h in range(8) for v in (0, 1)]
    vals = _pmap(lambda k: T.canon_rows(wl, k[0], k[1], k[2], k[3], 0, N64K), keys)
    return dict(zip(keys, vals))


def _run_64k(wl, fmt, tail, rows):
    cache = kvq.Cache(1, 8, 32, fmt, tail_tokens=tail, n_seqs=1, max_tokens=N64K)
    # ragged chunking: a long chunk, single tokens, and a remainder
    T.fill(cache, wl, 0, [0], 8, N64K, T.chunk_list(N64K, [20011, 1, 7, 12345]))
    q = T.query(wl, 0, 0, 0, 32, "cuda").unsqueeze(0)
    out = cache.decode(0, [0], q)
    torch.cuda.synchronize()
    n, n_q = cache.seq_get(0, 0)
    assert n == N64K and n_q == O.nq_after(0, N64K, tail, O.granule(O.FORMAT_NAMES.index(fmt), O.FORMAT_NAMES.index(fmt)))
    worst = _check_units(cache, fmt, wl, [(0, 0, h) for h in range(8)], rows,
                         {(0, 0): T.query_values(q)[0]}, {(0, 0): out[0].cpu().numpy()})
    del cache, out
    _release()
    return worst


@pytest.mark.parametrize("tail", [0, 1024, 2048])
@pytest.mark.parametrize("fmt", synth.WORKLOADS["c2_sweep_ctx65536"]["fmts"])
def test_sweep_64k_every_format_and_tail(fmt, tail, rows_c2):
    _run_64k("c2_sweep_ctx65536", fmt, tail, rows_c2)


@pytest.mark.parametrize("fmt", list(synth.WORKLOADS["c3_kvarn_ctx65536"]["fmts"]) + ["kvarn4_1"])
def test_kvarn_64k_tail_1024(fmt, rows_c3):
    _run_64k("c3_kvarn_ctx65536", fmt, 1024, rows_c3)


# --------------------------------------------------------------------------------------
# 240,000-token, 64-layer decode step (the benchmark's workload)

N240K = 240000
SAMPLED_LAYERS = (0, 31, 63)


@pytest.mark.parametrize("fmt", ["kvarn4", "q4_0"])
def test_decode_240k_64_layers_sampled(fmt):
    wl = "c4_ctx240000_64l"
    L, H = 64, 8
    cache = kvq.Cache(L, H, 32, fmt, tail_tokens=2048, n_seqs=1, max_tokens=N240K + 512)
    for layer in range(L):
        T.fill(cache, wl, 0, [layer], H, N240K, [16384] * 15)
    outs, qs = {}, {}
    for layer in range(L):
        q = T.query(wl, 0, layer, 0, 32, "cuda").unsqueeze(0)
        o = cache.decode(layer, [0], q)
        if layer in SAMPLED_LAYERS:
            outs[(0, layer)] = o[0].cpu().numpy()
            qs[(0, layer)] = T.query_values(q)[0]
    torch.cuda.synchronize()
    keys = [(0, l, h, v) for l in SAMPLED_LAYERS for h in range(H) for v in (0, 1)]
    rows = dict(zip(keys, _pmap(lambda k: T.canon_rows(wl, k[0], k[1], k[2], k[3], 0, N240K), keys)))
    _check_units(cache, fmt, wl, [(0, l, h) for l in SAMPLED_LAYERS for h in range(H)], rows, qs, outs)
    del cache, o
    _release()


# --------------------------------------------------------------------------------------
# Ragged batch: 16 sequences, 64 layers, kvarn3, tail 1024, 512-token append step

def _batch_input(wl, layers, H, spans):
    """K and V for `spans` [(seq, t0, t1)] concatenated along tokens: [len(layers)][sum][H][128]."""
    ks, vs = [], []
    for layer in layers:
        kl, vl = [], []
        for seq, t0, t1 in spans:
            k, v = T.layer_input(wl, seq, layer, H, t0, t1, "cuda")
            kl.append(k)
            vl.append(v)
        ks.append(torch.cat(kl, 0))
        vs.append(torch.cat(vl, 0))
    return torch.stack(ks, 0).contiguous(), torch.stack(vs, 0).contiguous()


def test_ragged_batch_16_sequences_64_layers():
    wl = "c5_ragged16_64l"
    w = synth.WORKLOADS[wl]
    fmt, tail, step = "kvarn3", w["tail"], w["chunk"]
    L, H, S = 64, 8, w["n_seqs"]
    lens = synth.seq_lengths(wl)
    cache = kvq.Cache(L, H, 32, fmt, tail_tokens=tail, n_seqs=S, max_tokens=max(lens) + step + 128)
    seqs = list(range(S))
    # fill: per layer, all sequences in one call per round of up to 8192 tokens each
    for layer in range(L):
        t = [0] * S
        while any(t[s] < lens[s] for s in seqs):
            spans = [(s, t[s], min(lens[s], t[s] + 8192)) for s in seqs if t[s] < lens[s]]
            k, v = _batch_input(wl, [layer], H, spans)
            cache.append(layer, [s for s, _, _ in spans], [b - a for _, a, b in spans], k[0], v[0])
            for s, a, b in spans:
                t[s] = b
    # decode step 0 (all sequences batched), then one 512-token append step on every layer
    sampled_seqs = (int(np.argmin(lens)), int(np.argmax(lens)), 7)
    sampled_layers = (0, 63)

    def decode_all(step_i):
        outs, qs = {}, {}
        for layer in range(L):
            q = torch.stack([T.query(wl, s, layer, step_i, 32, "cuda") for s in seqs], 0).contiguous()
            o = cache.decode(layer, seqs, q)
            if layer in sampled_layers:
                oc = o.cpu().numpy()
                qv = T.query_values(q)
                for s in sampled_seqs:
                    outs[(s, layer)] = oc[s]
                    qs[(s, layer)] = qv[s]
        torch.cuda.synchronize()
        return outs, qs

    outs0, qs0 = decode_all(0)
    k, v = _batch_input(wl, range(L), H, [(s, lens[s], lens[s] + step) for s in seqs])
    cache.append(-1, seqs, [step] * S, k, v)
    del k, v
    outs1, qs1 = decode_all(1)
    for s in seqs:
        n, n_q = cache.seq_get(s, 0)
        assert n == lens[s] + step and n_q == O.nq_after(0, n, tail, 128)
    units = [(s, l, h) for s in sampled_seqs for l in sampled_layers for h in (0, 5)]
    keys = [(s, l, h, vv) for s, l, h in units for vv in (0, 1)]
    rows = dict(zip(keys, _pmap(lambda kk: T.canon_rows(wl, kk[0], kk[1], kk[2], kk[3], 0, lens[kk[0]] + step), keys)))
    _check_units(cache, fmt, wl, units, rows, qs1, outs1)
    # decode before the append step: attention over the first lens[s] tokens, same encoder
    # state boundaries as the oracle's for that length
    for s, l, h in units[:4]:
        n0 = lens[s]
        n_q0 = O.nq_after(0, n0, tail, 128)
        r_k, r_v = rows[(s, l, h, 0)][:n0], rows[(s, l, h, 1)][:n0]
        ref = T.oracle_attention(fmt, r_k, r_v, n0, n_q0, qs0[(s, l)][h * 4:(h + 1) * 4], SIGMA)
        e = T.rel_err(outs0[(s, l)][h * 4:(h + 1) * 4], ref)
        assert e <= TOL, "step-0 attention seq %d layer %d head %d: %.3g" % (s, l, h, e)
    del cache
    _release()
