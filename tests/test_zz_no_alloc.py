"""kv_decode_attn_noalloc (no workspace, no allocation: the library's per-device array)
against kv_decode_attn through the C ABI, on two calls in a row, the second with a smaller
input; both also against the oracle (attention within 2e-3 normwise per head)."""
import math

import numpy as np
import pytest
import torch

from mixed_precision_quantized_amd import kvq

import kvq_testlib as T

pytestmark = pytest.mark.gpu
SIGMA = 1.0 / math.sqrt(128)


def _case(fmt, H, n, tail, chunks):
    wl = "c3_kvarn_ctx65536" if "kvarn" in fmt else "c2_sweep_ctx65536"
    cache = T.make_cache(fmt, 1, H, 4 * H, tail_tokens=tail, n_seqs=1, max_tokens=n)
    T.fill(cache, wl, 0, [0], H, n, T.chunk_list(n, chunks))
    q = T.query(wl, 0, 0, 0, 4 * H, "cuda").unsqueeze(0).contiguous()
    out_ws = cache.decode(0, [0], q)
    out_na = torch.full_like(out_ws, float("nan"))
    cache.decode_noalloc(0, [0], q, out_na)
    torch.cuda.synchronize()
    # the same kernels over the same split plan: identical results
    assert torch.equal(out_ws, out_na), "%s: the two entry points differ" % fmt
    n_, n_q = cache.seq_get(0, 0)
    qv = T.query_values(q)[0]
    got = out_na.cpu().numpy()[0]
    for h in (0, H - 1):
        k = T.canon_rows(wl, 0, 0, h, 0, 0, n)
        v = T.canon_rows(wl, 0, 0, h, 1, 0, n)
        ref = T.oracle_attention(fmt, k, v, n, n_q, qv[4 * h:4 * h + 4], SIGMA)
        assert T.rel_err(got[4 * h:4 * h + 4], ref) <= 2e-3


def test_noalloc_decode_two_calls_second_smaller():
    _case("kvarn4", 8, 9000, 300, [4000, 5000])
    _case("q4_0/q8_1", 2, 700, 100, [700])


def test_noalloc_errors():
    cache = kvq.Cache(1, 1, 4, "q4_0", tail_tokens=16, n_seqs=1, max_tokens=64)
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((1, 4, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KVError) as e:
        cache.decode_noalloc(0, [0], q, out)                # empty sequence
    assert e.value.code == kvq.KV_EEMPTY
    with pytest.raises(kvq.KVError) as e:
        cache.decode_noalloc(1, [0], q, out)                # bad layer
    assert e.value.code == kvq.KV_EINVAL
