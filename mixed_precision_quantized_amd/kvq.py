"""Python binding of libkvq.so (include/kvq.h): argument marshalling only.

Every step of the cache runs in the HIP kernels behind the C ABI; torch provides the
device memory and the stream.  There is no CPU fallback: if the library is not built,
`lib()` raises.

    cache = Cache(n_layers=1, n_kv_heads=8, n_q_heads=32, fmt="kvarn4", tail_tokens=1024,
                  n_seqs=1, max_tokens=65536)
    cache.append(layer=0, seq_ids=[0], n_new=[n], k=k_bf16, v=v_bf16)
    out = cache.decode(layer=0, seq_ids=[0], q=q)
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; KVQ_LIB_PATH may name another build of the same library (the HIP
# library either way: there is no CPU path)
LIB_PATH = os.environ.get("KVQ_LIB_PATH") or os.path.join(HERE, "libkvq.so")

FORMATS = ["bf16", "q2_0", "q2_1", "q3_0", "q3_1", "q4_0", "q4_1", "q5_0", "q5_1", "q6_0",
           "q6_1", "q8_0", "q8_1", "kvarn2", "kvarn3", "kvarn4", "kvarn5", "kvarn6", "kvarn8",
           "kvarn2_1", "kvarn3_1", "kvarn4_1", "kvarn5_1", "kvarn6_1", "kvarn8_1"]
FORMAT_ID = {n: i for i, n in enumerate(FORMATS)}

KV_OK, KV_EINVAL, KV_ENOSPC, KV_EUNSUPPORTED, KV_EEMPTY, KV_EDEVICE, KV_ESIZE = 0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "KV_OK", -1: "KV_EINVAL", -2: "KV_ENOSPC", -3: "KV_EUNSUPPORTED",
                -4: "KV_EEMPTY", -5: "KV_EDEVICE", -6: "KV_ESIZE"}
IN_BF16, IN_F32 = 0, 1


class KVError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__("%s failed: %s (%d)" % (what, STATUS_NAMES.get(code, "?"), code))
        self.code = code


class KVConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("fmt_k", ctypes.c_int32), ("fmt_v", ctypes.c_int32),
                ("tail_tokens", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64), ("tail_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_LIB = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def lib():
    """The loaded HIP library.  Raises RuntimeError if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkvq.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        cfgp = ctypes.POINTER(KVConfig)
        L.kv_cache_bytes.argtypes = [cfgp]
        L.kv_cache_bytes.restype = _i64
        L.kv_cache_init.argtypes = [cfgp, _vp, _i64, ctypes.POINTER(_vp)]
        L.kv_cache_init.restype = ctypes.c_int
        L.kv_cache_destroy.argtypes = [_vp]
        L.kv_cache_destroy.restype = ctypes.c_int
        L.kv_append.argtypes = [_vp, _i32, _i32, _i32p, _i32p, _vp, _vp, _i32, _vp]
        L.kv_append.restype = ctypes.c_int
        L.kv_decode_workspace_bytes.argtypes = [_vp, _i32]
        L.kv_decode_workspace_bytes.restype = _i64
        L.kv_decode_attn.argtypes = [_vp, _i32, _i32, _i32p, _vp, _i32, ctypes.c_float, _vp, _vp, _i64, _vp]
        L.kv_decode_attn.restype = ctypes.c_int
        L.kv_decode_attn_noalloc.argtypes = [_vp, _i32, _i32, _i32p, _vp, _i32, ctypes.c_float, _vp, _vp]
        L.kv_decode_attn_noalloc.restype = ctypes.c_int
        L.kv_prefill_workspace_bytes.argtypes = [_vp, _i32]
        L.kv_prefill_workspace_bytes.restype = _i64
        L.kv_prefill_attn.argtypes = [_vp, _i32, _i32, _i32, _vp, _i32, ctypes.c_float, _vp, _vp, _i64, _vp]
        L.kv_prefill_attn.restype = ctypes.c_int
        L.kv_attn_kld_workspace_bytes.argtypes = [_vp]
        L.kv_attn_kld_workspace_bytes.restype = _i64
        L.kv_attn_kld.argtypes = [_vp, _i32, _i32, _vp, _i32, ctypes.c_float, _vp, _vp, _vp, _i64, _vp]
        L.kv_attn_kld.restype = ctypes.c_int
        L.kv_spill_tail.argtypes = [_vp, _i32, _i32, _i32, _vp]
        L.kv_spill_tail.restype = ctypes.c_int
        L.kv_seq_get.argtypes = [_vp, _i32, _i32, _i64p, _i64p]
        L.kv_seq_get.restype = ctypes.c_int
        L.kv_seq_set.argtypes = [_vp, _i32, _i32, _i64, _i64]
        L.kv_seq_set.restype = ctypes.c_int
        L.kv_stream_layout.argtypes = [_vp, _i32, _i32, _i32, _i32, _i64p, _i64p]
        L.kv_stream_layout.restype = ctypes.c_int
        L.kv_format_info.argtypes = [_i32, _i32p, _i32p, _i32p, _i32p]
        L.kv_format_info.restype = ctypes.c_int
        L.kv_debug_convert.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, _vp]
        L.kv_debug_convert.restype = ctypes.c_int
        L.kv_debug_decode_events.argtypes = [_vp, _vp]
        L.kv_debug_decode_events.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _check(rc: int, what: str):
    if rc != KV_OK:
        raise KVError(rc, what)


def _ids(xs):
    arr = (ctypes.c_int32 * len(xs))(*[int(x) for x in xs])
    return arr


def _on(stream):
    """Allocation context for buffers a call on `stream` uses: torch's caching allocator
    then ties them to that stream, so a buffer freed after the call is reused only by work
    ordered after the kernels that read or write it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def fmt_id(f) -> int:
    return FORMAT_ID[f] if isinstance(f, str) else int(f)


def format_info(fmt):
    """(bits, code_bytes, scale_bytes, page_bytes) from the library's own table."""
    vals = [ctypes.c_int32() for _ in range(4)]
    _check(lib().kv_format_info(fmt_id(fmt), *[ctypes.byref(v) for v in vals]), "kv_format_info")
    return tuple(v.value for v in vals)


TAIL_DTYPES = {"bf16": 0, "f16": 1}


def make_config(n_layers, n_kv_heads, n_q_heads, fmt_k, fmt_v, tail_tokens, n_seqs, max_tokens,
                head_dim=128, tail_dtype="bf16") -> KVConfig:
    return KVConfig(n_layers, n_kv_heads, n_q_heads, head_dim, fmt_id(fmt_k), fmt_id(fmt_v),
                    tail_tokens, n_seqs, max_tokens, TAIL_DTYPES[tail_dtype], 0)


def cache_bytes(cfg: KVConfig) -> int:
    return int(lib().kv_cache_bytes(ctypes.byref(cfg)))


class Cache:
    """A cache over one caller-owned device buffer (a torch uint8 tensor)."""

    def __init__(self, n_layers, n_kv_heads, n_q_heads, fmt=None, tail_tokens=0, n_seqs=1,
                 max_tokens=4096, fmt_k=None, fmt_v=None, device="cuda", tail_dtype="bf16"):
        fk = fmt_k if fmt_k is not None else fmt
        fv = fmt_v if fmt_v is not None else fmt
        self.cfg = make_config(n_layers, n_kv_heads, n_q_heads, fk, fv, tail_tokens, n_seqs, max_tokens,
                               tail_dtype=tail_dtype)
        nbytes = cache_bytes(self.cfg)
        if nbytes < 0:
            raise KVError(nbytes, "kv_cache_bytes")
        self.nbytes = nbytes
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        _check(lib().kv_cache_init(ctypes.byref(self.cfg), ctypes.c_void_p(self.buf.data_ptr()),
                                   nbytes, ctypes.byref(h)), "kv_cache_init")
        self.h = h
        ws = int(lib().kv_decode_workspace_bytes(self.h, n_seqs))
        self.ws = torch.empty(ws, dtype=torch.uint8, device=device)

    def __del__(self):
        try:
            if getattr(self, "h", None) is not None and _LIB is not None:
                _LIB.kv_cache_destroy(self.h)
                self.h = None
        except Exception:
            pass

    # -- calls of the C ABI -------------------------------------------------------------
    def append(self, layer, seq_ids, n_new, k, v, stream=None):
        """k, v: device tensors [layers?][sum(n_new)][H][128], bfloat16 or float32."""
        assert k.dtype == v.dtype and k.is_contiguous() and v.is_contiguous()
        dt = IN_BF16 if k.dtype == torch.bfloat16 else IN_F32
        if k.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("k/v must be bfloat16 or float32")
        rc = lib().kv_append(self.h, int(layer), len(seq_ids), _ids(seq_ids), _ids(n_new),
                             ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()), dt,
                             _stream(stream))
        _check(rc, "kv_append")

    def decode(self, layer, seq_ids, q, softmax_scale=None, out=None, stream=None):
        """q: device [n_seqs][n_q_heads][128] bfloat16/float32 -> float32 output.  The
        cache's one decode workspace serves every call: calls on different streams must be
        ordered by the caller (events), as the C ABI requires."""
        assert q.is_contiguous()
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(128)
        if out is None:
            with _on(stream):
                out = torch.empty((len(seq_ids), self.cfg.n_q_heads, 128), dtype=torch.float32, device=q.device)
        dt = IN_BF16 if q.dtype == torch.bfloat16 else IN_F32
        rc = lib().kv_decode_attn(self.h, int(layer), len(seq_ids), _ids(seq_ids),
                                  ctypes.c_void_p(q.data_ptr()), dt, float(softmax_scale),
                                  ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(self.ws.data_ptr()),
                                  self.ws.numel(), _stream(stream))
        _check(rc, "kv_decode_attn")
        return out

    def decode_noalloc(self, layer, seq_ids, q, out, softmax_scale=None, stream=None):
        """decode() through kv_decode_attn_noalloc: no workspace, the library's own device
        array (calls on one device must not overlap); `out` is caller-provided."""
        assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(128)
        dt = IN_BF16 if q.dtype == torch.bfloat16 else IN_F32
        rc = lib().kv_decode_attn_noalloc(self.h, int(layer), len(seq_ids), _ids(seq_ids),
                                          ctypes.c_void_p(q.data_ptr()), dt, float(softmax_scale),
                                          ctypes.c_void_p(out.data_ptr()), _stream(stream))
        _check(rc, "kv_decode_attn_noalloc")
        return out

    def prefill(self, layer, seq_id, q, softmax_scale=None, out=None, ws=None, stream=None):
        """Causal attention of the sequence's last n_new tokens (already appended); q: device
        [n_new][n_q_heads][128] bfloat16/float32 -> float32 [n_new][n_q_heads][128]."""
        assert q.is_contiguous()
        n_new = q.shape[0]
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(128)
        if ws is None:
            n_ws = int(lib().kv_prefill_workspace_bytes(self.h, n_new))
            _check(n_ws if n_ws < 0 else 0, "kv_prefill_workspace_bytes")
            with _on(stream):
                ws = torch.empty(max(n_ws, 1), dtype=torch.uint8, device=q.device)
        if out is None:
            with _on(stream):
                out = torch.empty((n_new, self.cfg.n_q_heads, 128), dtype=torch.float32, device=q.device)
        dt = IN_BF16 if q.dtype == torch.bfloat16 else IN_F32
        rc = lib().kv_prefill_attn(self.h, int(layer), int(seq_id), n_new, ctypes.c_void_p(q.data_ptr()), dt,
                                   float(softmax_scale), ctypes.c_void_p(out.data_ptr()),
                                   ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream))
        _check(rc, "kv_prefill_attn")
        return out

    def attn_kld(self, layer, seq_id, q, k_ref, softmax_scale=None, stream=None):
        """KL(P || Q) per query head of the attention distributions over the exact keys
        (P; k_ref: device bfloat16 or int16 bits [n][n_kv_heads][128]) and over the keys the
        cache holds (Q).  q: device [n_q_heads][128] bfloat16/float32 -> float32 [n_q_heads]."""
        assert q.is_contiguous() and k_ref.is_contiguous() and k_ref.element_size() == 2
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(128)
        n_ws = int(lib().kv_attn_kld_workspace_bytes(self.h))
        _check(n_ws if n_ws < 0 else 0, "kv_attn_kld_workspace_bytes")
        with _on(stream):
            ws = torch.empty(max(n_ws, 1), dtype=torch.uint8, device=q.device)
            out = torch.empty(self.cfg.n_q_heads, dtype=torch.float32, device=q.device)
        dt = IN_BF16 if q.dtype == torch.bfloat16 else IN_F32
        rc = lib().kv_attn_kld(self.h, int(layer), int(seq_id), ctypes.c_void_p(q.data_ptr()), dt,
                               float(softmax_scale), ctypes.c_void_p(k_ref.data_ptr()),
                               ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                               ws.numel(), _stream(stream))
        _check(rc, "kv_attn_kld")
        return out

    def spill(self, layer, seq_id, keep_tokens, stream=None):
        _check(lib().kv_spill_tail(self.h, int(layer), int(seq_id), int(keep_tokens), _stream(stream)),
               "kv_spill_tail")

    def seq_get(self, seq, layer):
        n, nq = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().kv_seq_get(self.h, seq, layer, ctypes.byref(n), ctypes.byref(nq)), "kv_seq_get")
        return n.value, nq.value

    def seq_set(self, seq, layer, n, n_q):
        _check(lib().kv_seq_set(self.h, seq, layer, n, n_q), "kv_seq_set")

    def layout(self, seq, layer, head, is_v):
        offs = (ctypes.c_int64 * 4)()
        R = ctypes.c_int64()
        _check(lib().kv_stream_layout(self.h, seq, layer, head, is_v, offs, ctypes.byref(R)),
               "kv_stream_layout")
        return list(offs), R.value

    # -- inspection helpers (views into the device buffer) ---------------------------------
    def stream_views(self, seq, layer, head, is_v, n_q=None):
        """(codes [rows][code_bytes], scales [rows][halves] int16, cscale [pages][128] int16 or
        None, ring [R][128] int16) as device views; rows = n_q of (seq, layer)."""
        fmt = self.cfg.fmt_v if is_v else self.cfg.fmt_k
        bits, cb, sb, pb = format_info(fmt)
        (oc, os_, occ, orr), R = self.layout(seq, layer, head, is_v)
        if n_q is None:
            n_q = self.seq_get(seq, layer)[1]
        b = self.buf
        codes = b[oc: oc + n_q * cb].view(n_q, cb)
        scales = b[os_: os_ + n_q * sb].view(torch.int16).view(n_q, sb // 2) if sb else None
        cs = b[occ: occ + (n_q // 128) * 256].view(torch.int16).view(n_q // 128, 128) if occ >= 0 else None
        ring = b[orr: orr + R * 256].view(torch.int16).view(R, 128) if R else None
        return codes, scales, cs, ring


def debug_decode_events(before, after):
    """Bracket the split-K decode kernel of every following decode call with two
    torch.cuda.Event objects (recorded by the library on the call's stream, before the
    kernel and after it, ahead of the merge); debug_decode_events(None, None) clears it.
    The events are recorded once here first, so that their HIP handles exist."""
    if before is None and after is None:
        _check(lib().kv_debug_decode_events(None, None), "kv_debug_decode_events")
        return
    for e in (before, after):
        if not e.cuda_event:
            e.record()
    _check(lib().kv_debug_decode_events(ctypes.c_void_p(before.cuda_event), ctypes.c_void_p(after.cuda_event)),
           "kv_debug_decode_events")


def debug_convert(x: torch.Tensor):
    """Device conversions of a float32 CUDA tensor: (bf16 bits, fp16s bits, 1/x, sqrt x)."""
    assert x.dtype == torch.float32 and x.is_cuda and x.is_contiguous()
    n = x.numel()
    bo = torch.empty(n, dtype=torch.int16, device=x.device)
    ho = torch.empty(n, dtype=torch.int16, device=x.device)
    ro = torch.empty(n, dtype=torch.float32, device=x.device)
    so = torch.empty(n, dtype=torch.float32, device=x.device)
    rc = lib().kv_debug_convert(ctypes.c_void_p(x.data_ptr()), n, ctypes.c_void_p(bo.data_ptr()),
                                ctypes.c_void_p(ho.data_ptr()), ctypes.c_void_p(ro.data_ptr()),
                                ctypes.c_void_p(so.data_ptr()), _stream(None))
    _check(rc, "kv_debug_convert")
    return bo, ho, ro, so
