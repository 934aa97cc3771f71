"""The decode-kernel timing hook (kv_debug_decode_events) on the GPU: while it is set, a
decode call records the two caller events around its split-K kernel; the results are the
same as without the hook, the bracketed time is positive and at most that of the whole call
(events around it), and clearing the hook leaves later calls alone."""
import pytest
import torch

from mixed_precision_quantized_amd import kvq

import kvq_testlib as T

WL = "c2_sweep_ctx65536"


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["q4_0", "kvarn4"])
def test_events_bracket_the_decode_kernel(fmt):
    H, n = 2, 4000
    cache = kvq.Cache(1, H, 4 * H, fmt, tail_tokens=300, n_seqs=1, max_tokens=n)
    k, v = T.layer_input(WL, 0, 0, H, 0, n, "cuda")
    cache.append(0, [0], [n], k, v)
    q = T.query(WL, 0, 0, 0, 4 * H, "cuda").unsqueeze(0).contiguous()
    ref = cache.decode(0, [0], q).clone()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    kvq.debug_decode_events(a, b)
    try:
        for _ in range(3):
            c0.record(stream)
            out = cache.decode(0, [0], q)
            c1.record(stream)
            torch.cuda.synchronize()
            assert torch.equal(out, ref)
            kern, call = a.elapsed_time(b), c0.elapsed_time(c1)
            assert 0.0 < kern <= call
    finally:
        kvq.debug_decode_events(None, None)
    # cleared: the events are no longer recorded by decode calls
    torch.cuda.synchronize()
    before = a.elapsed_time(b)
    out = cache.decode(0, [0], q)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert a.elapsed_time(b) == before
