"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: codes, block scales, channel scales and live ring rows byte-identical to the oracle;
decode attention within 2e-3 normwise relative error per head (max over heads of
||o_gpu - o_ref||_inf / ||o_ref||_inf) against the oracle's binary64 attention over the
same dequantized values.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_quantized_amd import kvq, synth

import kvq_testlib as T

pytestmark = pytest.mark.gpu
TOL = 2e-3
SIGMA = 1.0 / math.sqrt(128)


def test_synth_gpu_generation_matches_cpu():
    for wl in ("c1_q4_0_ctx4096", "c3_kvarn_ctx65536"):
        for is_v in (0, 1):
            a = synth.kv_rows(wl, 0, 3, 1, is_v, 1000, 1300, "cuda").cpu()
            b = synth.kv_rows(wl, 0, 3, 1, is_v, 1000, 1300, "cpu")
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
            assert torch.equal(synth.to_bf16_bits(a.cuda()).cpu().view(torch.int16),
                               synth.to_bf16_bits(b).view(torch.int16))


def test_device_conversions_against_cpu():
    # every finite nonzero binary16 value: the reciprocal the encoders use
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h) & (h != 0)].astype(np.float32)
    # random fp32 patterns (finite), ties of both roundings, subnormals
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    hi = rng.integers(0, 0x7F7F, size=1 << 16).astype(np.uint32)
    ties = np.concatenate([((hi << 16) | 0x8000).view(np.float32), ((hi << 16) | 0x18000 >> 4).view(np.float32)])
    allh = np.arange(0, 0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((allh[:-1] + allh[1:]) / 2).astype(np.float32)
    xs = np.concatenate([h, x, ties, mids, -mids]).astype(np.float32)
    xs = xs[np.isfinite(xs)]
    bo, ho, ro, so = kvq.debug_convert(torch.from_numpy(xs).cuda())
    bo, ho = bo.cpu().numpy().view(np.uint16), ho.cpu().numpy().view(np.uint16)
    ro, so = ro.cpu().numpy(), so.cpu().numpy()
    ref_b = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bo, ref_b)
    with np.errstate(over="ignore"):
        hh = xs.astype(np.float16)
    hh = np.where(np.isinf(hh), np.sign(hh) * np.float16(65504), hh).astype(np.float16)
    hh = np.where(hh == 0, np.float16(0), hh).astype(np.float16)
    assert np.array_equal(ho, hh.view(np.uint16))
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        rr = np.float32(1.0) / xs
        ss = np.sqrt(xs)
    fin = np.isfinite(rr)
    assert np.array_equal(ro[fin].view(np.uint32), rr[fin].view(np.uint32))
    pos = xs >= 0
    assert np.array_equal(so[pos].view(np.uint32), ss[pos].view(np.uint32))


def _check_unit(cache, fmt, wl, seq, layer, head, n, q, group, tol=TOL):
    """Byte parity of K and V of one unit plus attention of its `group` query heads."""
    krows = T.canon_rows(wl, seq, layer, head, 0, 0, n)
    vrows = T.canon_rows(wl, seq, layer, head, 1, 0, n)
    T.compare_stream(cache, fmt, krows, seq, layer, head, 0)
    T.compare_stream(cache, fmt, vrows, seq, layer, head, 1)
    return krows, vrows


def _attn_check(cache, fmt, wl, seq, layer, heads, n, q, out, group, tol=TOL):
    n_, n_q = cache.seq_get(seq, layer)
    qv = T.query_values(q)[0]
    worst = 0.0
    for h in heads:
        krows = T.canon_rows(wl, seq, layer, h, 0, 0, n)
        vrows = T.canon_rows(wl, seq, layer, h, 1, 0, n)
        ref = T.oracle_attention(fmt, krows, vrows, n, n_q, qv[h * group:(h + 1) * group], SIGMA)
        got = out[0, h * group:(h + 1) * group].cpu().numpy()
        e = T.rel_err(got, ref)
        worst = max(worst, e)
        assert e <= tol, "attention %s layer %d head %d: rel err %.3g" % (fmt, layer, h, e)
    return worst


@pytest.mark.parametrize("chunks", ["all", 512, [1, 7, 300, 13]], ids=["all", "c512", "ragged"])
def test_c1_q4_0_fp32_input(chunks):
    wl = "c1_q4_0_ctx4096"
    n = 4096
    cache = kvq.Cache(1, 1, 4, "q4_0", tail_tokens=256, n_seqs=1, max_tokens=n)
    T.fill(cache, wl, 0, [0], 1, n, T.chunk_list(n, chunks))
    torch.cuda.synchronize()
    assert cache.seq_get(0, 0) == (n, n - 256)
    _check_unit(cache, "q4_0", wl, 0, 0, 0, n, None, 4)
    q = T.query(wl, 0, 0, 0, 4, "cuda")
    out = cache.decode(0, [0], q.unsqueeze(0))
    torch.cuda.synchronize()
    _attn_check(cache, "q4_0", wl, 0, 0, [0], n, q.unsqueeze(0), out, 4)


SMALL_FORMATS = list(kvq.FORMATS)


@pytest.mark.parametrize("fmt", SMALL_FORMATS)
def test_every_format_small(fmt):
    """Two KV heads, 8 query heads, several pages plus a ragged tail, bf16 inputs."""
    wl = "c3_kvarn_ctx65536" if fmt.startswith("kvarn") else "c2_sweep_ctx65536"
    n, Tt = 1000, 200
    cache = kvq.Cache(2, 2, 8, fmt, tail_tokens=Tt, n_seqs=1, max_tokens=1200)
    T.fill(cache, wl, 0, [0, 1], 2, n, T.chunk_list(n, [333, 1, 250]))
    torch.cuda.synchronize()
    for layer in (0, 1):
        for h in (0, 1):
            _check_unit(cache, fmt, wl, 0, layer, h, n, None, 4)
    q = T.query(wl, 0, 1, 0, 8, "cuda").unsqueeze(0)
    out = cache.decode(1, [0], q)
    torch.cuda.synchronize()
    _attn_check(cache, fmt, wl, 0, 1, [0, 1], n, q, out, 4)


# Key and value formats may differ (keys are often kept at more bits): every pairing of
# kinds, widths that differ, a KVarN stream beside a block or bf16 stream, and two KVarN
# widths (whole pages for both streams as soon as one of them is KVarN).
MIXED_PAIRS = ["q8_0/q4_0", "q4_0/q4_1", "q4_1/q4_0", "q6_1/q2_0", "bf16/q4_0", "q5_0/bf16",
               "kvarn4/q4_0", "q4_0/kvarn4", "kvarn8/kvarn3", "kvarn4/q8_0", "q3_1/kvarn5",
               "kvarn4/q4_1", "q4_1/kvarn4", "kvarn4_1/q4_0", "q4_1/kvarn3_1", "kvarn4_1/kvarn4",
               "kvarn8_1/kvarn2_1", "bf16/kvarn5_1"]


@pytest.mark.parametrize("fmt", MIXED_PAIRS)
def test_mixed_key_value_formats_small(fmt):
    """Same shape as the per-format test, with different key and value formats."""
    wl = "c3_kvarn_ctx65536" if "kvarn" in fmt else "c2_sweep_ctx65536"
    n, Tt = 1000, 200
    cache = T.make_cache(fmt, 2, 2, 8, tail_tokens=Tt, n_seqs=1, max_tokens=1200)
    T.fill(cache, wl, 0, [0, 1], 2, n, T.chunk_list(n, [333, 1, 250]))
    torch.cuda.synchronize()
    for layer in (0, 1):
        for h in (0, 1):
            _check_unit(cache, fmt, wl, 0, layer, h, n, None, 4)
    q = T.query(wl, 0, 1, 0, 8, "cuda").unsqueeze(0)
    out = cache.decode(1, [0], q)
    torch.cuda.synchronize()
    _attn_check(cache, fmt, wl, 0, 1, [0, 1], n, q, out, 4)


FAST_PAIRS = ["q4_0/q4_1", "q4_1/q4_0", "kvarn4/q4_0", "q4_0/kvarn4", "kvarn4/q4_1", "q4_1/kvarn4",
              "q8_0/q4_0", "q4_0/q8_0", "q8_1/q8_1", "kvarn8/q8_1", "q8_0/kvarn3", "q3_0/q3_1",
              "q3_1/kvarn3", "kvarn3/q3_0", "q2_0/q2_1", "q2_1/kvarn8", "kvarn2/kvarn2", "kvarn8/q2_0",
              "q5_0/q5_1", "q5_1/kvarn5", "kvarn5/q6_1", "q6_0/q6_0", "q6_1/kvarn6", "kvarn6/q5_0",
              "q6_0/q4_0", "q4_1/q6_1", "kvarn5/kvarn5"]


# kvarnN_1 (KVarN over the affine block quantizer): every width as keys and as values, alone
# and beside the other kinds (the value minima cross page boundaries; affine 8-bit keys)
KVARN1_PAIRS = ["kvarn4_1", "kvarn3_1/kvarn3_1", "kvarn2_1/q4_1", "q8_0/kvarn6_1", "kvarn8_1/kvarn4",
                "kvarn5_1/kvarn5_1", "kvarn6_1/q2_0", "q4_0/kvarn8_1", "kvarn4/kvarn2_1", "kvarn8_1/kvarn8_1"]


@pytest.mark.parametrize("fmt", FAST_PAIRS + KVARN1_PAIRS)
def test_fast_kernel_mixed_pairs_many_pages(fmt):
    """The fast kernel (every code width) with different key and value formats: 8
    KV heads, 24k tokens (many pages per pair of waves, a partial last page, a 1024-token
    tail), all heads checked."""
    wl = "c3_kvarn_ctx65536" if "kvarn" in fmt else "c2_sweep_ctx65536"
    n, Tt = 24000, 1024
    cache = T.make_cache(fmt, 1, 8, 32, tail_tokens=Tt, n_seqs=1, max_tokens=n)
    T.fill(cache, wl, 0, [0], 8, n, T.chunk_list(n, [7001, 1, 5000]))
    torch.cuda.synchronize()
    for h in (0, 7):
        _check_unit(cache, fmt, wl, 0, 0, h, n, None, 4)
    q = T.query(wl, 0, 0, 0, 32, "cuda").unsqueeze(0)
    out = cache.decode(0, [0], q)
    torch.cuda.synchronize()
    _attn_check(cache, fmt, wl, 0, 0, range(8), n, q, out, 4)


@pytest.mark.parametrize("fmt", ["q4_0", "q3_1", "kvarn4"])
def test_tail_covers_context_equals_bf16_attention(fmt):
    wl = "c2_sweep_ctx65536"
    n = 700
    cache = kvq.Cache(1, 1, 4, fmt, tail_tokens=1024, n_seqs=1, max_tokens=1024)
    T.fill(cache, wl, 0, [0], 1, n, [n])
    assert cache.seq_get(0, 0) == (n, 0)
    q = T.query(wl, 0, 0, 0, 4, "cuda").unsqueeze(0)
    out = cache.decode(0, [0], q).cpu().numpy()[0]
    k = T.canon_rows(wl, 0, 0, 0, 0, 0, n)
    v = T.canon_rows(wl, 0, 0, 0, 1, 0, n)
    K = (k.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    V = (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s = SIGMA * (T.query_values(q)[0] @ K.T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (p @ V) / p.sum(axis=1, keepdims=True)
    assert T.rel_err(out, ref) <= TOL


@pytest.mark.parametrize("fmt", ["q4_0", "q8_1", "kvarn3"])
def test_zero_tail_and_spill_equal_full_quantization(fmt):
    wl = "c2_sweep_ctx65536"
    n = 640
    full = kvq.Cache(1, 1, 4, fmt, tail_tokens=0, n_seqs=1, max_tokens=n)
    T.fill(full, wl, 0, [0], 1, n, [200, 440])
    tailed = kvq.Cache(1, 1, 4, fmt, tail_tokens=300, n_seqs=1, max_tokens=n)
    T.fill(tailed, wl, 0, [0], 1, n, [n])
    assert tailed.seq_get(0, 0)[1] < n
    tailed.spill(0, 0, 0)
    torch.cuda.synchronize()
    assert full.seq_get(0, 0) == (n, n) and tailed.seq_get(0, 0) == (n, n)
    for is_v in (0, 1):
        a = T.device_stream(full, 0, 0, 0, is_v)
        b = T.device_stream(tailed, 0, 0, 0, is_v)
        for x, y in zip(a[:3], b[:3]):
            if x is not None:
                assert np.array_equal(x, y)
        rows = T.canon_rows(wl, 0, 0, 0, is_v, 0, n)
        T.compare_stream(full, fmt, rows, 0, 0, 0, is_v)


def test_decode_reads_only_and_append_is_deterministic():
    wl = "c2_sweep_ctx65536"
    n = 900
    caches = []
    for _ in range(2):
        c = kvq.Cache(1, 2, 8, "kvarn4", tail_tokens=100, n_seqs=1, max_tokens=1024)
        c.buf.zero_()
        T.fill(c, wl, 0, [0], 2, n, [450, 450])
        caches.append(c)
    torch.cuda.synchronize()
    assert torch.equal(caches[0].buf, caches[1].buf)
    before = caches[0].buf.clone()
    q = T.query(wl, 0, 0, 0, 8, "cuda").unsqueeze(0)
    o1 = caches[0].decode(0, [0], q)
    for _ in range(3):
        o2 = caches[0].decode(0, [0], q)
    torch.cuda.synchronize()
    assert torch.equal(before, caches[0].buf)
    assert torch.allclose(o1, o2, rtol=0, atol=0)
