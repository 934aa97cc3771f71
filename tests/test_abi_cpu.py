"""Host-side checks of libkvq.so that need no GPU.

* the library loads and exports every function include/*.h declares;
* kv_cache_bytes reproduces the pages' memory arithmetic through the product's own
  format table and layout (256 B per BF16 vector, 64 KiB per 4-bit token at 64 layers x
  8 KV heads, ...);
* every validation path returns its status synchronously and enqueues nothing: the calls
  use a fake device address that is never dereferenced.
"""
import ctypes
import glob
import os
import re

import pytest

from mixed_precision_quantized_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000   # 256-byte aligned address that no device call ever sees here


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        txt = open(h).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        for m in re.finditer(r"^\s*(?:int|int64_t|void)\s+\**\s*(kv_\w+)\s*\(", txt, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = kvq.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n


def cfg(fmt="q4_0", L=1, H=1, QH=4, T=0, S=1, M=4096, fk=None, fv=None, D=128):
    return kvq.make_config(L, H, QH, fk or fmt, fv or fmt, T, S, M, head_dim=D)


def test_bytes_reproduce_page_arithmetic():
    # BF16 cache: 2 * 64 layers * 8 KV heads * 128 dims * 2 B = 262,144 B per token; the
    # ring of a bf16 stream is tiny against the 240,000-token rows.
    c = cfg("bf16", L=64, H=8, QH=32, T=0, M=240000)
    per_tok_rows = kvq.cache_bytes(c) / 240000
    assert abs(per_tok_rows - 262144) / 262144 < 1e-3
    # 4-bit codes: 64 KiB per token without scales; q4_0 adds 8 B of fp16 scales per vector
    c4 = cfg("q4_0", L=64, H=8, QH=32, T=0, M=240000)
    assert abs(kvq.cache_bytes(c4) / 240000 - 2 * 64 * 8 * 72) / (2 * 64 * 8 * 72) < 1e-3
    # the 1,024-token BF16 tail adds its ring: 1024 * 2 * 64 * 8 * 256 B = 0.25 GiB
    c4t = cfg("q4_0", L=64, H=8, QH=32, T=1024, M=240000)
    ring = kvq.cache_bytes(c4t) - kvq.cache_bytes(c4)
    assert abs(ring - 1024 * 262144) <= 2 * 64 * 8 * 256
    # kvarn4: 74 B per vector (64 codes + 8 scales + 2 amortized channel-scale bytes)
    ck = cfg("kvarn4", L=64, H=8, QH=32, T=0, M=240000)
    assert abs(kvq.cache_bytes(ck) / 240000 - 2 * 64 * 8 * 74) / (2 * 64 * 8 * 74) < 2e-3


def test_format_table_matches_sizes():
    sizes = {"q2_0": 40, "q2_1": 48, "q3_0": 56, "q3_1": 64, "q4_0": 72, "q4_1": 80,
             "q5_0": 88, "q5_1": 96, "q6_0": 104, "q6_1": 112, "q8_0": 136, "q8_1": 144,
             "kvarn2": 42, "kvarn3": 58, "kvarn4": 74, "kvarn5": 90, "kvarn6": 106,
             "kvarn8": 138, "kvarn2_1": 50, "kvarn3_1": 66, "kvarn4_1": 82, "kvarn5_1": 98,
             "kvarn6_1": 114, "kvarn8_1": 146, "bf16": 256}
    for name, b in sizes.items():
        bits, cb, sb, pb = kvq.format_info(name)
        assert cb + sb + pb // 128 == b


def test_config_validation():
    assert kvq.cache_bytes(cfg(D=64)) == kvq.KV_EUNSUPPORTED
    assert kvq.cache_bytes(cfg(QH=6, H=4)) == kvq.KV_EINVAL
    # K and V may use different formats: the cache holds one stream of each
    mixed = kvq.cache_bytes(cfg(fk="q8_0", fv="q4_0"))
    assert mixed > 0
    assert kvq.cache_bytes(cfg(fk="q8_0", fv="q8_0")) > mixed > kvq.cache_bytes(cfg(fk="q4_0", fv="q4_0"))
    assert kvq.cache_bytes(cfg(fk="kvarn4", fv="q4_0")) > 0
    assert kvq.cache_bytes(cfg(T=-1)) == kvq.KV_EINVAL
    assert kvq.cache_bytes(cfg(M=0)) == kvq.KV_EINVAL
    c = cfg()
    c.fmt_k = 99
    assert kvq.cache_bytes(c) == kvq.KV_EINVAL
    assert kvq.cache_bytes(cfg()) > 0


def _handle(c, nbytes=None):
    L = kvq.lib()
    h = ctypes.c_void_p()
    n = kvq.cache_bytes(c) if nbytes is None else nbytes
    rc = L.kv_cache_init(ctypes.byref(c), ctypes.c_void_p(FAKE), n, ctypes.byref(h))
    return rc, h


def test_init_errors():
    L = kvq.lib()
    c = cfg()
    rc, _ = _handle(c, kvq.cache_bytes(c) - 1)
    assert rc == kvq.KV_ESIZE
    h = ctypes.c_void_p()
    assert L.kv_cache_init(ctypes.byref(c), ctypes.c_void_p(FAKE + 8), kvq.cache_bytes(c), ctypes.byref(h)) == kvq.KV_EINVAL
    assert L.kv_cache_init(ctypes.byref(c), None, kvq.cache_bytes(c), ctypes.byref(h)) == kvq.KV_EINVAL
    rc, h = _handle(c)
    assert rc == kvq.KV_OK
    assert L.kv_cache_destroy(h) == 0


def test_append_decode_spill_validation_paths():
    L = kvq.lib()
    c = cfg(T=16, S=2, M=100)
    rc, h = _handle(c)
    assert rc == 0
    ids = kvq._ids([0])
    n = kvq._ids([101])
    ptr = ctypes.c_void_p(FAKE)
    # capacity
    assert L.kv_append(h, 0, 1, ids, n, ptr, ptr, 0, None) == kvq.KV_ENOSPC
    # bad layer, dtype, ids, negative count, null inputs
    assert L.kv_append(h, 1, 1, ids, kvq._ids([1]), ptr, ptr, 0, None) == kvq.KV_EINVAL
    assert L.kv_append(h, -2, 1, ids, kvq._ids([1]), ptr, ptr, 0, None) == kvq.KV_EINVAL
    assert L.kv_append(h, 0, 1, ids, kvq._ids([1]), ptr, ptr, 7, None) == kvq.KV_EINVAL
    assert L.kv_append(h, 0, 1, kvq._ids([2]), kvq._ids([1]), ptr, ptr, 0, None) == kvq.KV_EINVAL
    assert L.kv_append(h, 0, 2, kvq._ids([1, 1]), kvq._ids([1, 1]), ptr, ptr, 0, None) == kvq.KV_EINVAL
    assert L.kv_append(h, 0, 1, ids, kvq._ids([-1]), ptr, ptr, 0, None) == kvq.KV_EINVAL
    assert L.kv_append(h, 0, 1, ids, kvq._ids([1]), None, ptr, 0, None) == kvq.KV_EINVAL
    # zero tokens: nothing to do, succeeds without any device call
    assert L.kv_append(h, 0, 1, ids, kvq._ids([0]), None, None, 0, None) == kvq.KV_OK
    # nothing changed
    nn, nq = ctypes.c_int64(), ctypes.c_int64()
    assert L.kv_seq_get(h, 0, 0, ctypes.byref(nn), ctypes.byref(nq)) == 0 and nn.value == 0 and nq.value == 0
    # decode: empty sequence, bad scale, small workspace
    ws = L.kv_decode_workspace_bytes(h, 1)
    assert ws > 0
    assert L.kv_decode_attn(h, 0, 1, ids, ptr, 0, 0.1, ptr, ptr, ws, None) == kvq.KV_EEMPTY
    assert L.kv_decode_attn(h, 0, 1, ids, ptr, 0, 0.1, ptr, ptr, ws - 1, None) == kvq.KV_ESIZE
    assert L.kv_decode_attn(h, 0, 1, ids, ptr, 0, float("nan"), ptr, ptr, ws, None) == kvq.KV_EINVAL
    assert L.kv_decode_attn(h, 0, 1, ids, ptr, 5, 0.1, ptr, ptr, ws, None) == kvq.KV_EINVAL
    assert L.kv_decode_attn(h, 3, 1, ids, ptr, 0, 0.1, ptr, ptr, ws, None) == kvq.KV_EINVAL
    # the allocation-free entry point checks the same arguments before any device call
    assert L.kv_decode_attn_noalloc(h, 0, 1, ids, ptr, 0, 0.1, ptr, None) == kvq.KV_EEMPTY
    assert L.kv_decode_attn_noalloc(h, 3, 1, ids, ptr, 0, 0.1, ptr, None) == kvq.KV_EINVAL
    assert L.kv_decode_attn_noalloc(h, 0, 1, ids, None, 0, 0.1, ptr, None) == kvq.KV_EINVAL
    assert L.kv_decode_attn_noalloc(None, 0, 1, ids, ptr, 0, 0.1, ptr, None) == kvq.KV_EINVAL
    # spill: keep larger than the tail, bad seq
    assert L.kv_spill_tail(h, 0, 0, 17, None) == kvq.KV_EINVAL
    assert L.kv_spill_tail(h, 0, 5, 0, None) == kvq.KV_EINVAL
    # seq_set rules: n_q <= n <= max_tokens, occupancy within the ring
    assert L.kv_seq_set(h, 0, 0, 101, 0) == kvq.KV_EINVAL
    assert L.kv_seq_set(h, 0, 0, 10, 11) == kvq.KV_EINVAL
    assert L.kv_seq_set(h, 0, 0, 40, 0) == kvq.KV_EINVAL       # 40 > ring of 16
    assert L.kv_seq_set(h, 0, 0, 40, 30) == kvq.KV_OK
    assert L.kv_seq_get(h, 0, 0, ctypes.byref(nn), ctypes.byref(nq)) == 0 and (nn.value, nq.value) == (40, 30)
    assert L.kv_seq_set(h, 0, -1, 0, 0) == kvq.KV_OK
    L.kv_cache_destroy(h)


def test_kvarn_granule_rules():
    L = kvq.lib()
    c = cfg("kvarn3", T=100, M=1000)
    rc, h = _handle(c)
    assert rc == 0
    offs = (ctypes.c_int64 * 4)()
    R = ctypes.c_int64()
    assert L.kv_stream_layout(h, 0, 0, 0, 1, offs, ctypes.byref(R)) == 0
    assert R.value == 256                     # 128 * ceil((100 + 127) / 128)
    assert offs[2] > 0 and offs[1] > offs[0] and offs[3] > offs[2]
    assert L.kv_seq_set(h, 0, 0, 200, 100) == kvq.KV_EINVAL    # n_q must be a page multiple
    assert L.kv_seq_set(h, 0, 0, 200, 128) == kvq.KV_OK
    L.kv_cache_destroy(h)


def test_noalloc_rejects_plans_beyond_its_array():
    """kv_decode_attn_noalloc: a plan that cannot fit the library's 1024-partial device array
    (600 KV heads need at least 1200 workgroups) is rejected before any device call."""
    L = kvq.lib()
    c = cfg(H=600, QH=2400, M=256)
    rc, h = _handle(c)
    assert rc == 0
    assert L.kv_seq_set(h, 0, 0, 10, 10) == kvq.KV_OK       # 10 quantized tokens (tail 0)
    ids = kvq._ids([0])
    ptr = ctypes.c_void_p(FAKE)
    assert L.kv_decode_attn_noalloc(h, 0, 1, ids, ptr, 0, 0.1, ptr, None) == kvq.KV_ESIZE
    L.kv_cache_destroy(h)


def test_prefill_rejects_a_ring_beyond_32_bit_offsets():
    """The prefill reads the 16-bit ring through one buffer resource: a ring of 2^23 slots
    or more (2 GiB of rows per stream) is refused before any device call; the quantized
    rows need no such limit (their resources are rebased per block)."""
    L = kvq.lib()
    big = (1 << 23) + 10
    c = cfg("q4_0", T=big, M=big + 100)
    rc, h = _handle(c)
    assert rc == 0
    assert L.kv_seq_set(h, 0, 0, big, 0) == kvq.KV_OK
    n_ws = L.kv_prefill_workspace_bytes(h, 1)
    ptr = ctypes.c_void_p(FAKE)
    assert L.kv_prefill_attn(h, 0, 0, 1, ptr, 0, 0.1, ptr, ptr, n_ws, None) == kvq.KV_EUNSUPPORTED
    L.kv_cache_destroy(h)
    # a ring just under the limit passes validation (then fails only at the launch, which
    # this host never reaches: no device call is made for a validation error)
    c = cfg("q4_0", T=(1 << 23) - 1, M=(1 << 23) + 100)
    rc, h = _handle(c)
    assert rc == 0
    L.kv_cache_destroy(h)


def test_kv_log_prints_the_configuration():
    """KV_LOG=1 prints each cache's formats, tail, granule, ring and size at creation (to
    stderr); unset, the library prints nothing."""
    import subprocess
    import sys
    code = ("import ctypes; from mixed_precision_quantized_amd import kvq; "
            "c = kvq.make_config(2, 8, 32, 'kvarn4', 'q4_0', 1024, 3, 5000); h = ctypes.c_void_p(); "
            "print(kvq.lib().kv_cache_init(ctypes.byref(c), ctypes.c_void_p(%d), kvq.cache_bytes(c), "
            "ctypes.byref(h)))" % FAKE)
    env = dict(os.environ, KV_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "0", r.stderr[-2000:]
    line = [l for l in r.stderr.splitlines() if l.startswith("kvq: cache")]
    assert len(line) == 1, r.stderr
    for part in ("keys kvarn4", "values q4_0", "tail 1024 (bf16)", "granule 128", "2 layers x 8 KV heads x 32 q heads",
                 "3 sequences x 5000 tokens"):
        assert part in line[0], line[0]
    env.pop("KV_LOG")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT, timeout=120)
    assert "kvq:" not in r.stderr


def test_decode_events_hook_validation():
    # the measurement hook stores two caller event handles; it touches no device, so its
    # argument checks run here: exactly one null is refused, two nulls clear it
    L = kvq.lib()
    assert L.kv_debug_decode_events(ctypes.c_void_p(FAKE), None) == kvq.KV_EINVAL
    assert L.kv_debug_decode_events(None, ctypes.c_void_p(FAKE)) == kvq.KV_EINVAL
    assert L.kv_debug_decode_events(None, None) == kvq.KV_OK
