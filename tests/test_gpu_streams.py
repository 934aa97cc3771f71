"""Calls on a caller-supplied stream that is not torch's current stream (GPU): decode,
prefill and the KL harness enqueue on that stream, and buffers the binding allocates for
them are tied to it.  Results equal those of the same calls on the current stream."""
import pytest
import torch

from mixed_precision_quantized_amd import kvq

import kvq_testlib as T

WL = "c2_sweep_ctx65536"


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["q4_0", "kvarn4"])
def test_side_stream_results_match(fmt):
    H, n = 2, 1500
    cache = kvq.Cache(1, H, 4 * H, fmt, tail_tokens=200, n_seqs=1, max_tokens=n)
    k, v = T.layer_input(WL, 0, 0, H, 0, n, "cuda")
    cache.append(0, [0], [n], k, v)
    q = T.query(WL, 0, 0, 0, 4 * H, "cuda").unsqueeze(0).contiguous()
    qp = torch.stack([T.query(WL, 0, 0, i, 4 * H, "cuda") for i in range(40)], 0).contiguous()
    ref_d = cache.decode(0, [0], q).clone()
    ref_p = cache.prefill(0, 0, qp).clone()
    ref_k = cache.attn_kld(0, 0, q[0], k).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append((cache.decode(0, [0], q, stream=s), cache.prefill(0, 0, qp, stream=s),
                     cache.attn_kld(0, 0, q[0], k, stream=s)))
        # churn on the current stream meanwhile: freed blocks must not be handed to it
        junk = torch.empty(1 << 20, device="cuda").fill_(float("nan"))
        del junk
    s.synchronize()
    for d, p, kl in outs:
        assert torch.equal(d, ref_d)
        assert torch.equal(p, ref_p)
        assert torch.equal(kl, ref_k)
