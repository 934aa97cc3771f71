"""Benchmark of the quantized KV cache hot path on one MI355X.

Workload (default): 64 layers x 8 KV heads (32 query heads, GQA 4) x head_dim 128, one
sequence at 240,000 tokens of context, kvarn4 cache with a 2,048-token BF16 tail, seeded
synthetic bf16 K/V (Gaussian, 4 of 128 key channels x15).  A step is one pass of the whole
hot path: append one token to all 64 layers (canonicalize, ring write, spill the oldest
tail token, KVarN page encode every 128 steps) and decode attention on all 64 layers.

Reported (one JSON line):
  value      decode-attention KV read rate, GB/s: algorithmic bytes of the 64 decodes
             (every quantized row K+V plus every BF16 ring row, read once) / their time
  roofline   the decode kernel against HBM peak (8 TB/s), per launch from HIP events
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
  append     the ragged batch (16 sequences, lengths uniform on [8000, 120000], 64 layers,
             kvarn3, BF16 tail 1024): one step appends a 512-token chunk to every sequence on
             all 64 layers, then decodes all 64 layers for the 16 sequences.  Sequence-tokens
             per second with an HBM roof (826 B per stream-token) and an ALU co-roof (the page
             encoder's lane operations), and the ragged decode's KV read rate.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_hbm_traffic_kvarn4_ctx240000.md")
DECODE_SOURCES = ["kvq_decode_ws.h", "kvq_decode_ws_key.hip", "kvq_decode_ws.hip", "kvq_decode.hip",
                  "kvq_merge.hip", "kvq_host.cpp", "kvq_internal.h", "kvq_device.h"]


def measured_traffic(fmt, ctx, tail, kv_heads):
    """HBM bytes of one launch of the split-K decode kernel from the committed counter
    summary, or None when it does not cover this workload or the decode sources changed
    since it was taken."""
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "mixed_precision_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    want = {"fmt": fmt, "ctx": str(ctx), "tail": str(tail), "kv_heads": str(kv_heads),
            "sources_sha256": h.hexdigest()}
    for line in lines:
        parts = line.split()
        if parts[:1] != ["traffic_per_launch"]:
            continue
        kv = dict(x.split("=", 1) for x in parts[1:])
        if all(kv.get(k) == v for k, v in want.items()):
            return int(kv["bytes"])
    return None


APPEND_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "append_ragged16_kvarn3.md")
APPEND_SOURCES = ["kvq_append.hip", "kvq_host.cpp", "kvq_internal.h", "kvq_device.h"]


def measured_append_traffic():
    """HBM bytes of one 16-sequence append step from the committed counter summary, or None
    when the append sources changed since it was taken."""
    import hashlib
    h = hashlib.sha256()
    for f in APPEND_SOURCES:
        with open(os.path.join(ROOT, "mixed_precision_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    try:
        lines = open(APPEND_TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    for line in lines:
        parts = line.split()
        if parts[:1] != ["append_traffic_per_step"]:
            continue
        kv = dict(x.split("=", 1) for x in parts[1:])
        if kv.get("sources_sha256") == h.hexdigest():
            return int(kv["bytes"])
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--fmt", default="kvarn4", help="cache format, or KEY/VALUE formats (e.g. q8_0/q4_0)")
    p.add_argument("--ctx", type=int, default=240000)
    p.add_argument("--layers", type=int, default=64)
    p.add_argument("--tail", type=int, default=2048)
    p.add_argument("--tail-dtype", default="bf16", choices=["bf16", "f16"],
                   help="16-bit type of the precision tail (and of the values quantized from it)")
    p.add_argument("--append-chunk", type=int, default=512)
    p.add_argument("--append-reps", type=int, default=4)
    p.add_argument("--cpu-units", type=int, default=16, help="(layer, kv head) units of the CPU sample")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-ragged", action="store_true", help="skip the 16-sequence append + decode leg")
    p.add_argument("--ragged-steps", type=int, default=5)
    p.add_argument("--ragged-only", action="store_true", help="only the 16-sequence leg (its own JSON line)")
    p.add_argument("--prefill", type=int, default=0, metavar="CHUNK",
                   help="chunked-prefill attention: time a CHUNK-token chunk at the end of --ctx tokens")
    p.add_argument("--sweep", action="store_true",
                   help="context-depth series (decode + prefill) and the 64k format sweeps")
    p.add_argument("--kld", action="store_true",
                   help="attention-fidelity sweep: median KL over query heads, format x tail x context")
    p.add_argument("--copy-probe", type=int, default=0,
                   help="only run a plain device copy of this many bytes (counter calibration)")
    return p.parse_args()


def stream_bytes(fmt):
    from mixed_precision_quantized_amd import kvq
    bits, cb, sb, pb = kvq.format_info(fmt)
    return cb + sb + pb / 128.0


def split_fmt(fmt):
    """'q8_0/q4_0' -> ('q8_0', 'q4_0'); a single name is both streams' format."""
    fk, _, fv = fmt.partition("/")
    return fk, fv or fk


def decode_bytes_layer(fmt, n, n_q, heads):
    """Algorithmic bytes of one decode launch: every quantized row of K and V (codes,
    block scales, amortized channel scales) plus every BF16 ring row, read once."""
    fk, fv = split_fmt(fmt)
    return heads * (n_q * (stream_bytes(fk) + stream_bytes(fv)) + (n - n_q) * 2 * 256)


# Lane operations of the KVarN page encoder per stream-token (one 128-dim vector), counted
# from its definition: FWHT-128 (7 x 128 add/sub), squares (128), 8 Sinkhorn iterations of a
# row pass and a column pass (each a multiply and an add per element: 4 x 128), the
# reciprocal channel scaling (128) and the block encode (max, scale, round, clamp, pack:
# 5 x 128); per-row and per-column square roots and reciprocals are amortized over 128.
KVARN_OPS_PER_STREAM_TOKEN = 7 * 128 + 128 + 8 * 4 * 128 + 128 + 5 * 128
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz: single (not packed, not fused) lane operations/s
ALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9


def append_bytes_stream_token(fmt, tail, in_bytes=256):
    """Algorithmic HBM bytes per stream-token of a steady-state append: the input row, the
    ring write and the ring read when the token spills (both only with a tail), the encoded
    row (codes, block scales, amortized channel scales)."""
    ring = 2 * 256 if tail > 0 else 0
    return in_bytes + ring + stream_bytes(fmt)


def ragged_leg(args):
    """The 16-sequence ragged workload: fill, then steps of (512-token append on all 64 layers
    for every sequence, 64 batched decodes); append and decode timed apart with HIP events."""
    import torch
    from mixed_precision_quantized_amd import kvq, synth
    wl = "c5_ragged16_64l"
    w = synth.WORKLOADS[wl]
    fmt, tail, chunk, S = w["fmts"][0], w["tail"], w["chunk"], w["n_seqs"]
    L, H, QH = w["layers"], w["kv_heads"], w["q_heads"]
    lens = synth.seq_lengths(wl)
    nsteps = args.warmup + args.ragged_steps
    cache = kvq.Cache(L, H, QH, fmt, tail_tokens=tail, n_seqs=S, max_tokens=max(lens) + nsteps * chunk + 128)
    seqs = list(range(S))

    def rows(layer, spans):
        k = torch.cat([torch.stack([synth.kv_rows(wl, s, layer, h, 0, a, b, "cuda") for h in range(H)], 1)
                       for s, a, b in spans], 0)
        v = torch.cat([torch.stack([synth.kv_rows(wl, s, layer, h, 1, a, b, "cuda") for h in range(H)], 1)
                       for s, a, b in spans], 0)
        return synth.to_bf16_bits(k).contiguous(), synth.to_bf16_bits(v).contiguous()

    t0 = time.time()
    for layer in range(L):
        t = [0] * S
        while any(t[s] < lens[s] for s in seqs):
            spans = [(s, t[s], min(lens[s], t[s] + 16384)) for s in seqs if t[s] < lens[s]]
            k, v = rows(layer, spans)
            cache.append(layer, [s for s, _, _ in spans], [b - a for _, a, b in spans], k, v)
            for s, a, b in spans:
                t[s] = b
        if layer % 16 == 15:
            torch.cuda.synchronize()
            print("  ragged: filled layer %d" % layer, file=sys.stderr, flush=True)
    print("  ragged fill %.1f s, cache %.2f GiB" % (time.time() - t0, cache.nbytes / 2**30), file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    out = torch.empty((S, QH, 128), dtype=torch.float32, device="cuda")
    qs = [torch.stack([synth.to_bf16_bits(synth.q_rows(wl, s, l, 0, QH, "cuda")) for s in seqs], 0).contiguous()
          for l in range(L)]
    app_ms, dec_ms, dec_bytes = [], [], []
    for i in range(nsteps):
        # the step's input, [L][16 x 512][H][128] per stream (made before the timed region)
        spans = [(s, lens[s] + i * chunk, lens[s] + (i + 1) * chunk) for s in seqs]
        kv = [rows(l, spans) for l in range(L)]
        K = torch.stack([x[0] for x in kv], 0).contiguous()
        V = torch.stack([x[1] for x in kv], 0).contiguous()
        del kv
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        cache.append(-1, seqs, [chunk] * S, K, V)
        ev[1].record(stream)
        for l in range(L):
            cache.decode(l, seqs, qs[l], out=out)
        ev[2].record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            app_ms.append(ev[0].elapsed_time(ev[1]))
            dec_ms.append(ev[1].elapsed_time(ev[2]))
            b = 0.0
            for s in seqs:
                n, n_q = cache.seq_get(s, 0)
                b += L * decode_bytes_layer(fmt, n, n_q, H)
            dec_bytes.append(b)
        del K, V
    print("  ragged: %d steps done" % nsteps, file=sys.stderr, flush=True)
    a_ms = sum(app_ms) / len(app_ms)
    tokens = S * chunk
    tps = tokens / (a_ms * 1e-3)
    bst = append_bytes_stream_token(fmt, tail)
    streams = L * H * 2
    hbm_gbs = tokens * streams * bst / (a_ms * 1e-3) / 1e9
    ops = tokens * streams * KVARN_OPS_PER_STREAM_TOKEN if fmt.startswith("kvarn") else 0
    alu = ops / (a_ms * 1e-3)
    d_ms = sum(dec_ms) / len(dec_ms)
    d_gbs = sum(dec_bytes) / len(dec_bytes) / (d_ms * 1e-3) / 1e9
    del cache
    torch.cuda.empty_cache()
    return {
        "workload": "16 sequences (lengths uniform on [8000, 120000], seeded), 64 layers x 8 KV heads x 32 q heads "
                    "x d128, %s, BF16 tail %d; a step appends %d tokens to every sequence on all 64 layers"
                    % (fmt, tail, chunk),
        "lengths": lens, "steps": len(app_ms),
        "tokens_per_s": round(tps, 1), "unit": "sequence-tokens/s", "ms_per_step": round(a_ms, 4),
        "bytes_per_stream_token": bst, "bytes_per_sequence_token": bst * streams,
        "roofline": {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "traffic": measured_append_traffic(),
                     "kernel": "one 64-layer append call (ring write, spill, page encode)",
                     "bytes_per_step": int(tokens * streams * bst)},
        "alu_roof": {"bound": "alu", "achieved": round(alu / 1e12, 3), "peak": round(ALU_PEAK_LANE_OPS / 1e12, 3),
                     "unit": "T lane-ops/s", "frac": round(alu / ALU_PEAK_LANE_OPS, 4),
                     "ops_per_stream_token": KVARN_OPS_PER_STREAM_TOKEN if ops else 0},
        "ragged_decode": {"value": round(d_gbs, 1), "unit": "GB/s", "pct_of_hbm_peak": round(100 * d_gbs / HBM_PEAK_GBS, 2),
                          "ms_per_step": round(d_ms, 4), "bytes_per_step": int(sum(dec_bytes) / len(dec_bytes))},
    }


def copy_probe(nbytes):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "dispatches": 5}))


def fill_cache(cache, wl, layers, heads, ctx, chunk=16384):
    import torch
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from mixed_precision_quantized_amd import synth
    for layer in range(layers):
        t = 0
        while t < ctx:
            c = min(chunk, ctx - t)
            k = torch.stack([synth.kv_rows(wl, 0, layer, h, 0, t, t + c, "cuda") for h in range(heads)], 1)
            v = torch.stack([synth.kv_rows(wl, 0, layer, h, 1, t, t + c, "cuda") for h in range(heads)], 1)
            cache.append(layer, [0], [c], synth.to_bf16_bits(k).contiguous(), synth.to_bf16_bits(v).contiguous())
            t += c
        if layer % 16 == 15:
            torch.cuda.synchronize()
            print("  filled layer %d" % layer, file=sys.stderr, flush=True)


def cpu_baseline(fmt, wl, ctx, tail, units):
    """The oracle, untuned, on `units` full-context (layer, KV head) units in parallel:
    encode (append) then binary64 decode attention.  One thread per unit."""
    import numpy as np
    import oracle as O
    from mixed_precision_quantized_amd import synth
    fk, fv = (O.FORMAT_NAMES.index(x) for x in split_fmt(fmt))
    G = O.granule(fk, fv)
    n_q = O.nq_after(0, ctx, tail, G)
    cores = min(units, os.cpu_count() or 1, 16)
    units = cores
    work = [(u // 8, u % 8) for u in range(units)]
    data = {}

    def gen(i):
        layer, h = work[i]
        k = synth.bf16_as_u16(synth.to_bf16_bits(synth.kv_rows(wl, 0, layer, h, 0, 0, ctx)))
        v = synth.bf16_as_u16(synth.to_bf16_bits(synth.kv_rows(wl, 0, layer, h, 1, 0, ctx)))
        data[i] = [k, v, None, None]

    def enc(i):
        k, v = data[i][0], data[i][1]
        data[i][2] = O.encode_stream(fk, n_q, k)
        data[i][3] = O.encode_stream(fv, n_q, v)

    def att(i):
        layer, h = work[i]
        k, v, kq, vq = data[i]
        q = synth.q_rows(wl, 0, layer, 0, 32)[4 * h: 4 * h + 4].double().numpy()
        O.attention(ctx, n_q, fk, fv, kq, vq, k[n_q:], v[n_q:], q, 1.0 / math.sqrt(128))

    def run(fn):
        ths = [threading.Thread(target=fn, args=(i,)) for i in range(units)]
        t0 = time.perf_counter()
        for t in ths:
            t.start()
        for t in ths:
            t.join()
        return time.perf_counter() - t0

    run(gen)
    t_enc = run(enc)
    t_att = run(att)
    # the same unit alone on one core (no other thread running)
    t1 = time.perf_counter()
    att(0)
    t_one = time.perf_counter() - t1
    byts = units * decode_bytes_layer(fmt, ctx, n_q, 1)
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": round(byts / t_att / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "cpu_model": model, "nproc": os.cpu_count(),
        "usable_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
        "sample": "%d full-context (layer, KV head) units of the same workload (%d tokens, %s, tail %d), "
                  "one thread each: binary64 decode attention over the oracle's own encoding"
                  % (units, ctx, fmt, tail),
        "seconds": round(t_att, 2),
        "append_tokens_per_s": round(units * ctx / (64 * 8) / t_enc, 1),
        "append_seconds": round(t_enc, 2),
        "single_core": {"value": round(byts / units / t_one / 1e9, 4), "unit": "GB/s", "cores": 1,
                        "sample": "one of the same units, alone", "seconds": round(t_one, 2)},
    }


KLD_FMTS = ["q2_0", "q3_0", "q4_0", "q5_0", "q6_0", "q8_0", "kvarn2", "kvarn3", "kvarn4", "kvarn5",
            "kvarn6", "kvarn8"]


def kld_sweep(args):
    """Median over the 32 query heads of KL(P || Q) (attention over exact BF16 keys vs over the
    cache's keys) for every format of the pages' KLD table, tails 0 / 1024 / 2048 and contexts
    4k / 16k / 64k: one layer, 8 KV heads, synthetic keys of the 64k KVarN sweep workload
    (N(0,1) with four 15x channels), its seeded queries.  Also times the KL kernel."""
    import numpy as np
    import torch
    from mixed_precision_quantized_amd import kvq, synth
    wl, H, QH = "c3_kvarn_ctx65536", 8, 32
    ctxs = [4096, 16384, 65536]
    keys = torch.stack([synth.kv_rows(wl, 0, 0, h, 0, 0, max(ctxs), "cuda") for h in range(H)], 1)
    vals = torch.stack([synth.kv_rows(wl, 0, 0, h, 1, 0, max(ctxs), "cuda") for h in range(H)], 1)
    kb, vb = synth.to_bf16_bits(keys).contiguous(), synth.to_bf16_bits(vals).contiguous()
    q = synth.to_bf16_bits(synth.q_rows(wl, 0, 0, 0, QH, "cuda")).contiguous()
    stream = torch.cuda.current_stream()
    table = []
    for ctx in ctxs:
        k_ref = kb[:ctx].contiguous()
        for fmt in KLD_FMTS:
            for tail in (0, 1024, 2048):
                cache = kvq.Cache(1, H, QH, fmt, tail_tokens=tail, n_seqs=1, max_tokens=ctx)
                t = 0
                while t < ctx:
                    c = min(16384, ctx - t)
                    cache.append(0, [0], [c], kb[t:t + c].contiguous(), vb[t:t + c].contiguous())
                    t += c
                out = cache.attn_kld(0, 0, q, k_ref)
                a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a0.record(stream)
                for _ in range(3):
                    out = cache.attn_kld(0, 0, q, k_ref)
                a1.record(stream)
                torch.cuda.synchronize()
                us = a0.elapsed_time(a1) * 1e3 / 3
                n, n_q = cache.seq_get(0, 0)
                byts = H * (n_q * stream_bytes(fmt) + (n - n_q) * 256 + n * 256)
                kl = out.cpu().numpy().astype(np.float64)
                table.append({"ctx": ctx, "fmt": fmt, "tail": tail, "kld_median": float(np.median(kl)),
                              "kld_max": float(kl.max()), "us": round(us, 1),
                              "gbs": round(byts / (us * 1e-6) / 1e9, 1)})
                del cache
        print("  kld ctx %d done" % ctx, file=sys.stderr, flush=True)
    print(json.dumps({"metric": "attention KL divergence, median over query heads", "unit": "nats",
                      "data": "synthetic", "config": {"workload": "1 layer x 8 KV heads x 32 q heads x d128, "
                      "keys N(0,1) with four 15x channels, seeded queries, softmax scale 1/sqrt(128)"},
                      "table": table}), flush=True)


def prefill_bench(args):
    """Causal attention of a chunk of args.prefill tokens at the end of args.ctx tokens (one
    layer of the decode workload's shape: 8 KV heads, 32 query heads, the chosen format and
    tail), timed per call with HIP events.  Algorithmic work: for every query head and query
    i, 2 x 128 multiply-adds per visible key for q.k and as many for p.v."""
    import torch
    from mixed_precision_quantized_amd import kvq, synth
    wl, H, QH = "c4_ctx240000_64l", 8, 32
    n, c = args.ctx, args.prefill
    fk, fv = split_fmt(args.fmt)
    cache = kvq.Cache(1, H, QH, fmt_k=fk, fmt_v=fv, tail_tokens=args.tail, n_seqs=1, max_tokens=n)
    spans, t = [], 0
    while t < n - c:                       # the context, then the chunk as one append
        spans.append((t, min(t + 16384, n - c)))
        t = spans[-1][1]
    spans.append((n - c, n))
    for t0, t1 in spans:
        k = torch.stack([synth.kv_rows(wl, 0, 0, h, 0, t0, t1, "cuda") for h in range(H)], 1)
        v = torch.stack([synth.kv_rows(wl, 0, 0, h, 1, t0, t1, "cuda") for h in range(H)], 1)
        cache.append(0, [0], [t1 - t0], synth.to_bf16_bits(k).contiguous(), synth.to_bf16_bits(v).contiguous())
    q = torch.stack([synth.to_bf16_bits(synth.q_rows(wl, 0, 0, i, QH, "cuda")) for i in range(c)], 0).contiguous()
    n_ws = int(kvq.lib().kv_prefill_workspace_bytes(cache.h, c))
    ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
    out = torch.empty((c, QH, 128), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        cache.prefill(0, 0, q, out=out, ws=ws)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a0, a1 in evs:
        a0.record(stream)
        cache.prefill(0, 0, q, out=out, ws=ws)
        a1.record(stream)
    torch.cuda.synchronize()
    ms = sum(a0.elapsed_time(a1) for a0, a1 in evs) / args.steps
    visible = sum(n - c + i + 1 for i in range(c))
    flops = 4.0 * 128 * QH * visible
    tf = flops / (ms * 1e-3) / 1e12
    print(json.dumps({"metric": "chunked-prefill attention, chunk tokens/s per layer", "value": round(c / (ms * 1e-3), 1),
                      "unit": "tokens/s", "ms_per_call": round(ms, 4), "higher_is_better": True, "data": "synthetic",
                      "dtype": "f32", "operands": "f16 MFMA operands (exact codes, two-term query), f32 accumulate",
                      "config": {"workload": "1 layer x 8 KV heads x 32 q heads x d128, chunk %d at the end of %d "
                                             "tokens, %s, tail %d" % (c, n, args.fmt, args.tail)},
                      "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": 2500.0, "unit": "TFLOP/s",
                                   "frac": round(tf / 2500.0, 4), "traffic": None,
                                   "kernel": "k_prefill + k_prefill_merge", "flops_per_call": flops}}), flush=True)


def _fill_layers(cache, wl, L, H, ctx):
    import torch
    from mixed_precision_quantized_amd import synth
    for layer in range(L):
        t = 0
        while t < ctx:
            c = min(16384, ctx - t)
            k = torch.stack([synth.kv_rows(wl, 0, layer, h, 0, t, t + c, "cuda") for h in range(H)], 1)
            v = torch.stack([synth.kv_rows(wl, 0, layer, h, 1, t, t + c, "cuda") for h in range(H)], 1)
            cache.append(layer, [0], [c], synth.to_bf16_bits(k).contiguous(), synth.to_bf16_bits(v).contiguous())
            t += c


def _decode_rate(cache, wl, fmt, L, H, QH, reps=3):
    """Mean decode launch time over `reps` rounds of the L replica layers (events around the
    whole round), and the KV read rate from the algorithmic bytes."""
    import torch
    from mixed_precision_quantized_amd import synth
    qs = [synth.to_bf16_bits(synth.q_rows(wl, 0, l, 0, QH, "cuda")).unsqueeze(0).contiguous() for l in range(L)]
    out = torch.empty((1, QH, 128), dtype=torch.float32, device="cuda")
    for l in range(L):
        cache.decode(l, [0], qs[l], out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        for l in range(L):
            cache.decode(l, [0], qs[l], out=out)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (reps * L)
    n, n_q = cache.seq_get(0, 0)
    byts = decode_bytes_layer(fmt, n, n_q, H)
    return us, byts / (us * 1e-6) / 1e9


def _replicas(fmt, ctx, tail, H, G, floor_bytes=512e6, cap=64):
    """Layers of one workload, each a replica of the same shape, so that one round of
    decodes reads at least floor_bytes (more than the 256 MB last-level cache holds)."""
    n_q = max(0, (ctx - tail) // G * G)
    b = decode_bytes_layer(fmt, ctx, n_q, H)
    return int(min(cap, max(1, math.ceil(floor_bytes / b))))


def sweep(args):
    """Context-depth series (decode and chunked prefill, kvarn4 and q4_0, tail 2048, 4k to
    240k) and the 64k format sweeps (9 qN formats x tails 0 / 1024 / 2048 on Gaussian keys;
    kvarn2/3/4 x tail 1024 on Student-t keys), one layer shape (8 KV heads, 32 q heads),
    replicated over layers so that a round of decodes reads at least 512 MB."""
    import torch
    from mixed_precision_quantized_amd import kvq, synth
    H, QH = 8, 32
    depth, c2, c3 = [], [], []
    for fmt in ("kvarn4", "q4_0"):
        for ctx in (4096, 16384, 32768, 65536, 131072, 240000):
            tail = 2048
            G = 128 if fmt.startswith("kvarn") else 1
            L = _replicas(fmt, ctx, tail, H, G)
            cache = kvq.Cache(L, H, QH, fmt, tail_tokens=tail, n_seqs=1, max_tokens=ctx)
            _fill_layers(cache, "c4_ctx240000_64l", L, H, ctx)
            us, gbs = _decode_rate(cache, "c4_ctx240000_64l", fmt, L, H, QH)
            row = {"fmt": fmt, "ctx": ctx, "tail": tail, "replicas": L, "decode_us": round(us, 2),
                   "decode_gbs": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
            # chunked prefill: the last 512 tokens as the chunk, per layer
            c = 512
            q = torch.stack([synth.to_bf16_bits(synth.q_rows("c4_ctx240000_64l", 0, 0, i, QH, "cuda"))
                             for i in range(c)], 0).contiguous()
            ws = torch.empty(int(kvq.lib().kv_prefill_workspace_bytes(cache.h, c)), dtype=torch.uint8, device="cuda")
            pout = torch.empty((c, QH, 128), dtype=torch.float32, device="cuda")
            cache.prefill(0, 0, q, out=pout, ws=ws)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            stream = torch.cuda.current_stream()
            a.record(stream)
            for l in range(L):
                cache.prefill(l, 0, q, out=pout, ws=ws)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / L
            visible = sum(ctx - c + i + 1 for i in range(c))
            tf = 4.0 * 128 * QH * visible / (ms * 1e-3) / 1e12
            row.update({"prefill_chunk": c, "prefill_ms": round(ms, 4), "prefill_tokens_per_s": round(c / (ms * 1e-3), 1),
                        "prefill_tflops": round(tf, 1), "prefill_pct_of_f16_peak": round(100 * tf / 2500.0, 2)})
            depth.append(row)
            print("  sweep depth %s %d: %s GB/s" % (fmt, ctx, row["decode_gbs"]), file=sys.stderr, flush=True)
            del cache, ws, pout, q
            torch.cuda.empty_cache()
    for wl, fmts, tails, out in (("c2_sweep_ctx65536", synth.WORKLOADS["c2_sweep_ctx65536"]["fmts"], (0, 1024, 2048), c2),
                                  ("c3_kvarn_ctx65536", ("kvarn2", "kvarn3", "kvarn4"), (1024,), c3)):
        ctx = 65536
        for fmt in fmts:
            for tail in tails:
                G = 128 if fmt.startswith("kvarn") else 1
                L = _replicas(fmt, ctx, tail, H, G)
                cache = kvq.Cache(L, H, QH, fmt, tail_tokens=tail, n_seqs=1, max_tokens=ctx)
                _fill_layers(cache, wl, L, H, ctx)
                us, gbs = _decode_rate(cache, wl, fmt, L, H, QH)
                out.append({"fmt": fmt, "tail": tail, "replicas": L, "decode_us": round(us, 2),
                            "decode_gbs": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)})
                print("  sweep %s %s tail %d: %s GB/s" % (wl, fmt, tail, out[-1]["decode_gbs"]), file=sys.stderr,
                      flush=True)
                del cache
                torch.cuda.empty_cache()
        print("  sweep %s done" % wl, file=sys.stderr, flush=True)
    print(json.dumps({"metric": "decode KV read GB/s and chunked-prefill rate over context depth; 64k format sweeps",
                      "data": "synthetic", "device": torch.cuda.get_device_name(0),
                      "config": {"workload": "1 layer shape x 8 KV heads x 32 q heads x d128, batch 1, replicated over "
                                             "layers so that one round of decodes reads >= 512 MB"},
                      "depth": depth, "c2_sweep_64k": c2, "c3_kvarn_64k": c3}), flush=True)


def main():
    args = parse()
    if args.kld:
        kld_sweep(args)
        return
    if args.sweep:
        sweep(args)
        return
    if args.prefill:
        prefill_bench(args)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d)." % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.ragged_only:
        print(json.dumps({"metric": "ragged append sequence-tokens/s; ragged decode KV read GB/s",
                          "data": "synthetic", "append": ragged_leg(args)}), flush=True)
        return
    import torch
    from mixed_precision_quantized_amd import kvq, synth

    wl = "c4_ctx240000_64l"
    L, H, QH = args.layers, 8, 32
    steps, warm = args.steps, args.warmup
    extra = warm + steps + args.append_chunk * args.append_reps + 256
    print("bench: %s, %d layers, ctx %d, tail %d, %s" % (args.fmt, L, args.ctx, args.tail,
          torch.cuda.get_device_name(0)), file=sys.stderr, flush=True)
    fk, fv = split_fmt(args.fmt)
    cache = kvq.Cache(L, H, QH, fmt_k=fk, fmt_v=fv, tail_tokens=args.tail, n_seqs=1, max_tokens=args.ctx + extra,
                      tail_dtype=args.tail_dtype)
    t0 = time.time()
    fill_cache(cache, wl, L, H, args.ctx)
    torch.cuda.synchronize()
    print("  fill %.1f s, cache %.2f GiB" % (time.time() - t0, cache.nbytes / 2**30), file=sys.stderr, flush=True)

    qs = [synth.to_bf16_bits(synth.q_rows(wl, 0, l, 0, QH, "cuda")).unsqueeze(0).contiguous() for l in range(L)]
    out = torch.empty((1, QH, 128), dtype=torch.float32, device="cuda")
    tok_k = [synth.to_bf16_bits(torch.stack([synth.kv_rows(wl, 0, l, h, 0, args.ctx, args.ctx + extra, "cuda")
                                             for h in range(H)], 1)) for l in range(L)]
    tok_v = [synth.to_bf16_bits(torch.stack([synth.kv_rows(wl, 0, l, h, 1, args.ctx, args.ctx + extra, "cuda")
                                             for h in range(H)], 1)) for l in range(L)]
    K_all = torch.stack(tok_k, 0).contiguous()     # [L][extra][H][128]
    V_all = torch.stack(tok_v, 0).contiguous()
    del tok_k, tok_v
    stream = torch.cuda.current_stream()
    pos = [0]

    def step(ev_dec=None):
        # append one token to every layer (layer = -1: input [L][1][H][128])
        i = pos[0]
        cache.append(-1, [0], [1], K_all[:, i:i + 1].contiguous(), V_all[:, i:i + 1].contiguous())
        pos[0] += 1
        if ev_dec is not None:
            ev_dec[0].record(stream)
        for l in range(L):
            cache.decode(l, [0], qs[l], out=out)
        if ev_dec is not None:
            ev_dec[1].record(stream)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    dec_bytes = 0.0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(steps):
        step(evs[s])
        n, n_q = cache.seq_get(0, 0)
        dec_bytes += L * decode_bytes_layer(args.fmt, n, n_q, H)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t_start.elapsed_time(t_end) / steps
    dec_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    value = dec_bytes / steps / (dec_ms * 1e-3) / 1e9

    # per-launch duration of the split-K decode kernel alone: the library records a pair of
    # events on the call's stream right before and right after that kernel (ahead of the
    # merge), one pair per layer; also the whole call (events around it)
    n, n_q = cache.seq_get(0, 0)
    per, calls = [], []
    for l in range(L):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        kvq.debug_decode_events(a, b)
        c0.record(stream)
        cache.decode(l, [0], qs[l], out=out)
        c1.record(stream)
        kvq.debug_decode_events(None, None)
        per.append((a, b))
        calls.append((c0, c1))
    torch.cuda.synchronize()
    launch_ms = sum(a.elapsed_time(b) for a, b in per) / L
    call_ms = sum(a.elapsed_time(b) for a, b in calls) / L
    launch_bytes = decode_bytes_layer(args.fmt, n, n_q, H)
    achieved = launch_bytes / (launch_ms * 1e-3) / 1e9

    # append throughput: 512-token chunks into all 64 layers (layer = -1)
    ch = args.append_chunk
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start = pos[0]
    a0.record(stream)
    for r in range(args.append_reps):
        i = start + r * ch
        cache.append(-1, [0], [ch], K_all[:, i:i + ch].contiguous(), V_all[:, i:i + ch].contiguous())
    a1.record(stream)
    torch.cuda.synchronize()
    app_tps = ch * args.append_reps / (a0.elapsed_time(a1) * 1e-3)

    del cache, K_all, V_all
    torch.cuda.empty_cache()
    ragged = None if args.no_ragged else ragged_leg(args)

    cpu = None
    if not args.no_cpu:
        print("  cpu baseline ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.fmt, wl, args.ctx, args.tail, args.cpu_units)

    line = {
        "metric": "decode-attn KV read GB/s (% of HBM peak) @240k ctx; append tokens/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "operands": "i8 (scores) and f16 (values) MFMA operands, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "decode step, 64 layers x 8 KV heads x 32 q heads x d128, ctx %d, %s, "
                               "BF16 tail %d, batch 1" % (args.ctx, args.fmt, args.tail),
                   "layers": L, "kv_heads": H, "q_heads": QH, "ctx": args.ctx, "fmt": args.fmt,
                   "tail": args.tail, "batch": 1},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_ms_per_step": round(dec_ms, 4),
        "append_tokens_per_s": ragged["tokens_per_s"] if ragged else None,
        "append": ragged,
        "append_single_seq_tokens_per_s": round(app_tps, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.fmt, args.ctx, args.tail, H),
                     "kernel": "split-K decode kernel (%s), timed alone by events the library records around it"
                               % args.fmt,
                     "bytes_per_launch": int(launch_bytes), "launch_us": round(launch_ms * 1e3, 2),
                     "call_us": round(call_ms * 1e3, 2),
                     "call_frac": round(launch_bytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
