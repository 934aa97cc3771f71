// kvq_host.cpp -- host side of the C ABI declared in include/kvq.h.
//
// Host-only translation unit: argument validation, buffer sizing and layout, the
// precision-tail state machine and the decode split planner.  It contains no device
// code and calls the HIP runtime only through the launchers of kvq_internal.h, so every
// validation path runs (and is tested) on a machine without a GPU.
//
// Tail state machine ("Экспериментальные методы квантизации KV-кэша в BeeLLama.cpp
// v0.4.0: KVarN и precision tail", section "Как это работает: гибридное хранение
// кэша": the last T tokens stay BF16, positions before them use the low-bit type):
//   granule G = 128 if a stream is KVarN (whole pages are encoded at once), else 1;
//   after an append n += n_new and n_q = max(n_q, G*floor(max(0, n - T)/G));
//   after a spill with keep tokens n_q = max(n_q, G*floor(max(0, n - keep)/G));
//   token p with n_q <= p < n lives in ring slot p mod R, R = G*ceil((T+G-1)/G).
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

using namespace kvq;

struct kv_cache {
    kv_config cfg;
    CacheGeom geom;
    int64_t granule;
    int64_t ring_slots;
    int64_t max_tokens_pad;
    int64_t bytes;
    std::vector<int64_t> n;    // [seq * n_layers + layer]
    std::vector<int64_t> nq;
};

static_assert(KV_NUM_FORMATS == kNumFormats, "format count of the C ABI and the kernels");

namespace {

bool format_desc(int32_t fmt, FormatDesc* d)
{
    static const int8_t bits[KV_NUM_FORMATS] = {16, 2, 2, 3, 3, 4, 4, 5, 5, 6, 6, 8, 8,
                                                      2, 3, 4, 5, 6, 8, 2, 3, 4, 5, 6, 8};
    if (fmt < 0 || fmt >= KV_NUM_FORMATS) return false;
    FormatDesc r;
    r.bits = bits[fmt];
    if (fmt == KV_BF16) r.kind = KIND_BF16;
    else if (fmt >= KV_KVARN2_1) r.kind = KIND_KVARN1;
    else if (fmt >= KV_KVARN2) r.kind = KIND_KVARN;
    else r.kind = ((fmt - KV_Q2_0) % 2 == 0) ? KIND_Q0 : KIND_Q1;
    r.code_bytes = (r.kind == KIND_BF16) ? 256 : 16 * r.bits;
    r.scale_bytes = (r.kind == KIND_BF16) ? 0 : (kind_affine(r.kind) ? 16 : 8);
    r.page_bytes = kind_paged(r.kind) ? 256 : 0;
    *d = r;
    return true;
}

inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

StreamLayout stream_layout(const FormatDesc& f, int64_t tokens_pad, int64_t ring_slots)
{
    StreamLayout s;
    int64_t off = 0;
    s.codes = off;
    off = align256(off + tokens_pad * f.code_bytes);
    s.scales = off;
    off = align256(off + tokens_pad * f.scale_bytes);
    if (kind_paged(f.kind)) {
        s.cscale = off;
        off = align256(off + (tokens_pad / kPage) * 256);
    } else {
        s.cscale = -1;
    }
    s.ring = off;
    off = align256(off + ring_slots * 256);
    s.bytes = off;
    return s;
}

int64_t granule_of(int32_t fk, int32_t fv)
{
    FormatDesc a, b;
    format_desc(fk, &a);
    format_desc(fv, &b);
    return (kind_paged(a.kind) || kind_paged(b.kind)) ? kPage : 1;
}

int64_t ring_capacity(int64_t T, int64_t G) { return G * ((T + G - 1 + G - 1) / G); }

int64_t nq_after(int64_t nq, int64_t n, int64_t keep, int64_t G)
{
    int64_t over = std::max<int64_t>(0, n - keep);
    return std::max(nq, G * (over / G));
}

// Validates a configuration; fills the geometry (without base pointer) and total bytes.
// KV_LOG (environment): 1 prints each cache's configuration at creation, 2 also every
// decode call's split plan, to stderr.
int log_level()
{
    static const int level = [] {
        const char* e = std::getenv("KV_LOG");
        return e ? std::atoi(e) : 0;
    }();
    return level;
}

const char* format_name(int f)
{
    static const char* const names[KV_NUM_FORMATS] = {
        "bf16", "q2_0", "q2_1", "q3_0", "q3_1", "q4_0", "q4_1", "q5_0", "q5_1", "q6_0", "q6_1",
        "q8_0", "q8_1", "kvarn2", "kvarn3", "kvarn4", "kvarn5", "kvarn6", "kvarn8", "kvarn2_1",
        "kvarn3_1", "kvarn4_1", "kvarn5_1", "kvarn6_1", "kvarn8_1"};
    return f >= 0 && f < KV_NUM_FORMATS ? names[f] : "?";
}

int plan_config(const kv_config* cfg, CacheGeom* geom, int64_t* total, int64_t* G,
                int64_t* R, int64_t* tok_pad)
{
    if (!cfg) return KV_EINVAL;
    if (cfg->n_layers < 1 || cfg->n_kv_heads < 1 || cfg->n_q_heads < 1 || cfg->n_seqs < 1 ||
        cfg->max_tokens < 1 || cfg->tail_tokens < 0)
        return KV_EINVAL;
    if (cfg->n_q_heads % cfg->n_kv_heads) return KV_EINVAL;
    if (cfg->tail_dtype != KV_TAIL_BF16 && cfg->tail_dtype != KV_TAIL_F16) return KV_EINVAL;
    if (cfg->tail_dtype == KV_TAIL_F16 && (cfg->fmt_k == KV_BF16 || cfg->fmt_v == KV_BF16)) return KV_EUNSUPPORTED;
    FormatDesc fk, fv;
    if (!format_desc(cfg->fmt_k, &fk) || !format_desc(cfg->fmt_v, &fv)) return KV_EINVAL;
    if (cfg->head_dim != kD) return KV_EUNSUPPORTED;
    int group = cfg->n_q_heads / cfg->n_kv_heads;
    if (group > kMaxGroup) return KV_EUNSUPPORTED;
    // decode kernels are built for GQA groups of 4
    if (group != 4) return KV_EUNSUPPORTED;
    if (cfg->max_tokens > (int64_t(1) << 31) - kPage) return KV_EINVAL;
    int64_t g = granule_of(cfg->fmt_k, cfg->fmt_v);
    // The ring never holds more than min(T + G - 1, n) tokens, so a ring larger than the
    // capacity rounded up to G is never needed.
    int64_t r = std::min(ring_capacity(cfg->tail_tokens, g), ((cfg->max_tokens + g - 1) / g) * g);
    int64_t tp = ((cfg->max_tokens + kPage - 1) / kPage) * kPage;
    CacheGeom gm;
    std::memset(&gm, 0, sizeof(gm));
    gm.k = stream_layout(fk, tp, r);
    gm.v = stream_layout(fv, tp, r);
    gm.v_offset = gm.k.bytes;
    gm.unit_bytes = gm.k.bytes + gm.v.bytes;
    gm.fmt_k = cfg->fmt_k;
    gm.fmt_v = cfg->fmt_v;
    gm.n_layers = cfg->n_layers;
    gm.n_kv_heads = cfg->n_kv_heads;
    gm.n_q_heads = cfg->n_q_heads;
    gm.group = group;
    gm.ring_slots = (int32_t)r;
    gm.tail_f16 = cfg->tail_dtype == KV_TAIL_F16 ? 1 : 0;
    double units = (double)cfg->n_seqs * cfg->n_layers * cfg->n_kv_heads;
    if (units * (double)gm.unit_bytes > 9.0e18) return KV_EINVAL;
    if (geom) *geom = gm;
    if (total) *total = (int64_t)units * gm.unit_bytes;
    if (G) *G = g;
    if (R) *R = r;
    if (tok_pad) *tok_pad = tp;
    return KV_OK;
}

inline int64_t& n_at(kv_cache* c, int s, int l) { return c->n[(size_t)s * c->cfg.n_layers + l]; }
inline int64_t& nq_at(kv_cache* c, int s, int l) { return c->nq[(size_t)s * c->cfg.n_layers + l]; }

bool distinct_valid_ids(const kv_cache* c, int32_t n_seqs, const int32_t* ids)
{
    if (!ids || n_seqs < 1 || n_seqs > c->cfg.n_seqs) return false;
    std::vector<char> seen(c->cfg.n_seqs, 0);
    for (int i = 0; i < n_seqs; ++i) {
        if (ids[i] < 0 || ids[i] >= c->cfg.n_seqs || seen[ids[i]]) return false;
        seen[ids[i]] = 1;
    }
    return true;
}

// Enqueue the encode launches for one group of at most kMaxSeqsPerLaunch sequences.
int launch_group(kv_cache* c, AppendArgs& a, void* stream)
{
    FormatDesc fk, fv;
    format_desc(c->cfg.fmt_k, &fk);
    format_desc(c->cfg.fmt_v, &fv);
    bool any_enc = false, any_ring = false;
    for (int i = 0; i < a.n_seqs; ++i) {
        const AppendSeq& s = a.seqs[i];
        if (s.nq_new > s.nq_old) any_enc = true;
        if (s.n_new > std::max(s.nq_new, s.n_old)) any_ring = true;
    }
    int rc = 0;
    if (any_enc) {
        if (!kind_paged(fk.kind) || !kind_paged(fv.kind)) {
            rc = launch_append_encode(a, stream);
            if (rc) return rc;
        }
        if (kind_paged(fk.kind) || kind_paged(fv.kind)) {
            rc = launch_append_kvarn(a, stream);
            if (rc) return rc;
        }
    }
    // ring writes strictly after the encoders, which may read the slots being reused
    if (any_ring) rc = launch_append_ring(a, stream);
    return rc;
}

// Shared body of kv_append and kv_spill_tail once every argument is validated.
// entries: per sequence (seq, rows before it, n_new tokens); keep: T or keep_tokens.
int do_append(kv_cache* c, int32_t layer, int n_seqs, const int32_t* seqs, const int32_t* n_add,
              const void* k, const void* v, int32_t in_dtype, int64_t keep, void* stream)
{
    const int L = c->cfg.n_layers;
    const int l0 = layer < 0 ? 0 : layer;
    const int l1 = layer < 0 ? L : layer + 1;
    int64_t rows = 0;
    for (int i = 0; i < n_seqs; ++i) rows += n_add[i];
    std::vector<int64_t> new_n((size_t)n_seqs), new_nq((size_t)n_seqs);
    for (int i = 0; i < n_seqs; ++i) {
        int64_t n0 = n_at(c, seqs[i], l0);
        new_n[i] = n0 + n_add[i];
        new_nq[i] = nq_after(nq_at(c, seqs[i], l0), new_n[i], keep, c->granule);
    }
    // One launch set per layer range: when layer == -1 every layer of a sequence has the
    // same (n, n_q), so the per-sequence entries hold for all layers.
    for (int base = 0; base < n_seqs; base += kMaxSeqsPerLaunch) {
        AppendArgs a;
        std::memset(&a, 0, sizeof(a));
        a.g = c->geom;
        a.k_in = k;
        a.v_in = v;
        a.in_dtype = in_dtype;
        a.layer0 = l0;
        a.layers_in = l1 - l0;
        a.rows = (int32_t)rows;
        int cnt = std::min(kMaxSeqsPerLaunch, n_seqs - base);
        a.n_seqs = cnt;
        int64_t row0 = 0;
        for (int i = 0; i < base; ++i) row0 += n_add[i];
        for (int i = 0; i < cnt; ++i) {
            int j = base + i;
            AppendSeq& s = a.seqs[i];
            s.seq = seqs[j];
            s.in_row0 = (int32_t)row0;
            s.n_old = n_at(c, seqs[j], l0);
            s.n_new = new_n[j];
            s.nq_old = nq_at(c, seqs[j], l0);
            s.nq_new = new_nq[j];
            row0 += n_add[j];
        }
        int rc = launch_group(c, a, stream);
        if (rc) {
            // metadata advances anyway: the launches before the failure may have run
            for (int i = 0; i < n_seqs; ++i)
                for (int l = l0; l < l1; ++l) { n_at(c, seqs[i], l) = new_n[i]; nq_at(c, seqs[i], l) = new_nq[i]; }
            return KV_EDEVICE;
        }
    }
    for (int i = 0; i < n_seqs; ++i)
        for (int l = l0; l < l1; ++l) {
            n_at(c, seqs[i], l) = new_n[i];
            nq_at(c, seqs[i], l) = new_nq[i];
        }
    return KV_OK;
}

bool layers_agree(kv_cache* c, int32_t seq)
{
    for (int l = 1; l < c->cfg.n_layers; ++l)
        if (n_at(c, seq, l) != n_at(c, seq, 0) || nq_at(c, seq, l) != nq_at(c, seq, 0)) return false;
    return true;
}

}  // namespace

extern "C" {

int kv_format_info(int32_t fmt, int32_t* bits, int32_t* code_bytes, int32_t* scale_bytes,
                   int32_t* page_bytes)
{
    FormatDesc d;
    if (!format_desc(fmt, &d)) return KV_EINVAL;
    if (bits) *bits = d.bits;
    if (code_bytes) *code_bytes = d.code_bytes;
    if (scale_bytes) *scale_bytes = d.scale_bytes;
    if (page_bytes) *page_bytes = d.page_bytes;
    return KV_OK;
}

int64_t kv_cache_bytes(const kv_config* cfg)
{
    int64_t total = 0;
    int rc = plan_config(cfg, nullptr, &total, nullptr, nullptr, nullptr);
    return rc ? rc : total;
}

int kv_cache_init(const kv_config* cfg, void* dev_mem, int64_t bytes, kv_cache** out)
{
    if (!out) return KV_EINVAL;
    *out = nullptr;
    CacheGeom g;
    int64_t total, G, R, tp;
    int rc = plan_config(cfg, &g, &total, &G, &R, &tp);
    if (rc) return rc;
    if (!dev_mem || ((uintptr_t)dev_mem & 255)) return KV_EINVAL;
    if (bytes < total) return KV_ESIZE;
    kv_cache* c = new (std::nothrow) kv_cache;
    if (!c) return KV_EINVAL;
    c->cfg = *cfg;
    g.base = (char*)dev_mem;
    c->geom = g;
    c->granule = G;
    c->ring_slots = R;
    c->max_tokens_pad = tp;
    c->bytes = total;
    size_t cells = (size_t)cfg->n_seqs * cfg->n_layers;
    c->n.assign(cells, 0);
    c->nq.assign(cells, 0);
    if (log_level() >= 1)
        std::fprintf(stderr,
                     "kvq: cache keys %s values %s, tail %d (%s), granule %lld, ring %lld slots, %d layers x "
                     "%d KV heads x %d q heads, %d sequences x %lld tokens, %lld bytes\n",
                     format_name(cfg->fmt_k), format_name(cfg->fmt_v), cfg->tail_tokens,
                     cfg->tail_dtype == KV_TAIL_F16 ? "f16" : "bf16", (long long)G, (long long)R, cfg->n_layers,
                     cfg->n_kv_heads, cfg->n_q_heads, cfg->n_seqs, (long long)cfg->max_tokens, (long long)total);
    *out = c;
    return KV_OK;
}

int kv_cache_destroy(kv_cache* c)
{
    delete c;
    return KV_OK;
}

int kv_append(kv_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
              const int32_t* n_new, const void* k, const void* v, int32_t in_dtype, void* stream)
{
    if (!c || !n_new) return KV_EINVAL;
    if (layer < -1 || layer >= c->cfg.n_layers) return KV_EINVAL;
    if (in_dtype != KV_IN_BF16 && in_dtype != KV_IN_F32) return KV_EINVAL;
    if (!distinct_valid_ids(c, n_seqs, seq_ids)) return KV_EINVAL;
    int64_t rows = 0;
    for (int i = 0; i < n_seqs; ++i) {
        if (n_new[i] < 0) return KV_EINVAL;
        rows += n_new[i];
    }
    if (rows > (int64_t(1) << 30)) return KV_EINVAL;
    if (rows > 0 && (!k || !v)) return KV_EINVAL;
    const int l0 = layer < 0 ? 0 : layer;
    for (int i = 0; i < n_seqs; ++i) {
        if (layer < 0 && !layers_agree(c, seq_ids[i])) return KV_EINVAL;
        if (n_at(c, seq_ids[i], l0) + n_new[i] > c->cfg.max_tokens) return KV_ENOSPC;
    }
    if (rows == 0) return KV_OK;
    return do_append(c, layer, n_seqs, seq_ids, n_new, k, v, in_dtype, c->cfg.tail_tokens, stream);
}

int kv_spill_tail(kv_cache* c, int32_t layer, int32_t seq_id, int32_t keep_tokens, void* stream)
{
    if (!c) return KV_EINVAL;
    if (layer < -1 || layer >= c->cfg.n_layers) return KV_EINVAL;
    if (seq_id < 0 || seq_id >= c->cfg.n_seqs) return KV_EINVAL;
    if (keep_tokens < 0 || keep_tokens > c->cfg.tail_tokens) return KV_EINVAL;
    if (layer < 0) {
        // layers may differ here: spill each layer on its own
        if (!layers_agree(c, seq_id)) {
            for (int l = 0; l < c->cfg.n_layers; ++l) {
                int rc = kv_spill_tail(c, l, seq_id, keep_tokens, stream);
                if (rc) return rc;
            }
            return KV_OK;
        }
    }
    int32_t zero = 0;
    return do_append(c, layer, 1, &seq_id, &zero, nullptr, nullptr, KV_IN_BF16, keep_tokens, stream);
}

int64_t kv_decode_workspace_bytes(const kv_cache* c, int32_t n_seqs)
{
    if (!c || n_seqs < 1 || n_seqs > c->cfg.n_seqs) return KV_EINVAL;
    return align256((int64_t)kMaxDecodeWGs * kPartialFloats * 4);
}

namespace {
// Split plan of one prefill call: workgroups = KV heads x query tiles x key splits, about
// two per CU; quantized and ring blocks never share a split.
struct PfPlan { int32_t tiles, splits_q, splits_t, bps, bps_t, splits_max; };
PfPlan prefill_plan(const kv_cache* c, int64_t n, int64_t n_q, int32_t n_new)
{
    PfPlan p;
    p.tiles = (n_new + kPfQ - 1) / kPfQ;
    const int64_t nbq = (n_q + kPfKB - 1) / kPfKB, nbt = (n - n_q + kPfKB - 1) / kPfKB;
    const int64_t target = 2 * (int64_t)std::max(1, device_cu_count());
    const int64_t per = (int64_t)c->cfg.n_kv_heads * p.tiles;
    const int64_t splits = std::max<int64_t>(1, (target + per - 1) / per);
    p.bps = (int32_t)std::max<int64_t>(1, (nbq + nbt + splits - 1) / splits);
    p.splits_q = (int32_t)((nbq + p.bps - 1) / p.bps);
    // the ring region (a few thousand tokens) is its own launch: spread it as widely
    p.bps_t = (int32_t)std::max<int64_t>(1, (nbt + splits - 1) / splits);
    p.splits_t = (int32_t)((nbt + p.bps_t - 1) / p.bps_t);
    p.splits_max = (int32_t)(2 * splits + 2);
    return p;
}
}  // namespace

int64_t kv_prefill_workspace_bytes(const kv_cache* c, int32_t n_new)
{
    if (!c || n_new < 1) return KV_EINVAL;
    const PfPlan p = prefill_plan(c, c->cfg.max_tokens, 0, n_new);
    return align256((int64_t)c->cfg.n_kv_heads * p.tiles * p.splits_max * 4 * kPfQ * (kD + 2) * 4);
}

int kv_prefill_attn(kv_cache* c, int32_t layer, int32_t seq_id, int32_t n_new, const void* q,
                    int32_t q_dtype, float softmax_scale, float* out, void* workspace,
                    int64_t ws_bytes, void* stream)
{
    if (!c || layer < 0 || layer >= c->cfg.n_layers) return KV_EINVAL;
    if (seq_id < 0 || seq_id >= c->cfg.n_seqs) return KV_EINVAL;
    if (!q || !out || !workspace) return KV_EINVAL;
    if (q_dtype != KV_IN_BF16 && q_dtype != KV_IN_F32) return KV_EINVAL;
    if (!(softmax_scale == softmax_scale) || softmax_scale > 3.0e38f || softmax_scale < -3.0e38f)
        return KV_EINVAL;
    const int64_t n = n_at(c, seq_id, layer);
    if (n == 0) return KV_EEMPTY;
    if (n_new < 1 || n_new > n) return KV_EINVAL;
    if (ws_bytes < kv_prefill_workspace_bytes(c, n_new)) return KV_ESIZE;
    // the ring is read through one buffer resource with 32-bit offsets
    if (c->ring_slots * 256 >= (int64_t(1) << 31)) return KV_EUNSUPPORTED;
    PrefillArgs a;
    std::memset(&a, 0, sizeof(a));
    a.g = c->geom;
    a.layer = layer;
    a.seq = seq_id;
    a.n = n;
    a.n_q = nq_at(c, seq_id, layer);
    a.n_new = n_new;
    a.q_dtype = q_dtype;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    const PfPlan p = prefill_plan(c, a.n, a.n_q, n_new);
    a.tiles = p.tiles;
    a.splits_q = p.splits_q;
    a.splits_t = p.splits_t;
    a.bps = p.bps;
    a.bps_t = p.bps_t;
    if (p.splits_q + p.splits_t > p.splits_max) return KV_EUNSUPPORTED;   // the workspace's bound
    a.q = q;
    a.out = out;
    a.partials = (float*)workspace;
    return launch_prefill(a, stream) ? KV_EDEVICE : KV_OK;
}

int64_t kv_attn_kld_workspace_bytes(const kv_cache* c)
{
    if (!c) return KV_EINVAL;
    const int64_t splits = (c->cfg.max_tokens + kKldTokens - 1) / kKldTokens;
    return align256(splits * c->cfg.n_kv_heads * kMaxGroup * 4 * 4) + align256(c->cfg.n_q_heads * 4);
}

int kv_attn_kld(kv_cache* c, int32_t layer, int32_t seq_id, const void* q, int32_t q_dtype,
                float softmax_scale, const void* k_ref, float* kld, void* workspace,
                int64_t ws_bytes, void* stream)
{
    if (!c || layer < 0 || layer >= c->cfg.n_layers) return KV_EINVAL;
    if (seq_id < 0 || seq_id >= c->cfg.n_seqs) return KV_EINVAL;
    if (!q || !k_ref || !kld || !workspace) return KV_EINVAL;
    if (q_dtype != KV_IN_BF16 && q_dtype != KV_IN_F32) return KV_EINVAL;
    if (!(softmax_scale == softmax_scale) || softmax_scale > 3.0e38f || softmax_scale < -3.0e38f)
        return KV_EINVAL;
    if (ws_bytes < kv_attn_kld_workspace_bytes(c)) return KV_ESIZE;
    const int64_t n = n_at(c, seq_id, layer);
    if (n == 0) return KV_EEMPTY;
    KldArgs a;
    std::memset(&a, 0, sizeof(a));
    a.g = c->geom;
    a.layer = layer;
    a.seq = seq_id;
    a.n = n;
    a.n_q = nq_at(c, seq_id, layer);
    a.q_dtype = q_dtype;
    a.scale = softmax_scale;
    a.splits = (int32_t)((n + kKldTokens - 1) / kKldTokens);
    a.q = q;
    a.k_ref = (const uint16_t*)k_ref;
    a.partials = (float*)workspace;
    const int64_t splits_max = (c->cfg.max_tokens + kKldTokens - 1) / kKldTokens;
    a.cref = (float*)((char*)workspace + align256(splits_max * c->cfg.n_kv_heads * kMaxGroup * 4 * 4));
    a.out = kld;
    return launch_kld(a, stream) ? KV_EDEVICE : KV_OK;
}

}  // extern "C"

namespace {

// Argument checks shared by the decode entry points (everything but the workspace).
int decode_check(kv_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const void* q,
                 int32_t q_dtype, float softmax_scale, const float* out)
{
    if (!c || layer < 0 || layer >= c->cfg.n_layers) return KV_EINVAL;
    if (!distinct_valid_ids(c, n_seqs, seq_ids)) return KV_EINVAL;
    if (n_seqs > kMaxSeqsPerLaunch) return KV_EUNSUPPORTED;
    if (!q || !out) return KV_EINVAL;
    if (q_dtype != KV_IN_BF16 && q_dtype != KV_IN_F32) return KV_EINVAL;
    if (!(softmax_scale == softmax_scale) || softmax_scale > 3.0e38f || softmax_scale < -3.0e38f)
        return KV_EINVAL;
    return KV_OK;
}

int decode_nonempty(kv_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids)
{
    for (int i = 0; i < n_seqs; ++i)
        if (n_at(c, seq_ids[i], layer) == 0) return KV_EEMPTY;
    return KV_OK;
}

// Split plan (at most max_wgs workgroups, each leaving one partial) and launch of a checked
// decode call; `partials` holds max_wgs partials.  KV_EUNSUPPORTED if even the smallest plan
// (one quantized and one ring split per sequence and KV head) needs more.
int decode_launch(kv_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const void* q,
                  int32_t q_dtype, float softmax_scale, float* out, void* partials, int64_t max_wgs,
                  void* stream)
{
    DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.g = c->geom;
    a.layer = layer;
    a.n_seqs = n_seqs;
    a.q_dtype = q_dtype;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.q = q;
    a.out = out;
    a.partials = (float*)partials;
    const int H = c->cfg.n_kv_heads;
    int64_t total_units = 0, max_uq = 1, max_ut = 1;
    for (int i = 0; i < n_seqs; ++i) {
        DecodeSeq& s = a.seqs[i];
        s.seq = seq_ids[i];
        s.in_idx = i;
        s.n = n_at(c, seq_ids[i], layer);
        s.n_q = nq_at(c, seq_ids[i], layer);
        s.units_q = (int32_t)((s.n_q + kPage - 1) / kPage);
        s.units_t = (int32_t)((s.n - s.n_q + kTailUnit - 1) / kTailUnit);
        total_units += (int64_t)H * (4 * s.units_q + 5 * s.units_t);
        max_uq = std::max<int64_t>(max_uq, s.units_q);
        max_ut = std::max<int64_t>(max_ut, s.units_t);
    }
    // Balanced split.  Ring units and quantized pages never share a workgroup, so every
    // (sequence, KV head) needs one workgroup of each kind at least; while those are few
    // (at most an eighth of the resident workgroups) the grid is one resident wave, else up
    // to 4 waves of smaller splits, which the hardware hands out as workgroups finish (the
    // ring splits come last and fill the end).  A 32-token ring unit (16 KB of BF16 rows,
    // binary32 arithmetic) takes about 1.25 times as long as a 128-token quantized page, so
    // ring workgroups get 0.8 as many units (up to 0.9x when that saves a workgroup).
    int cus = device_cu_count();
    int per_cu = decode_wgs_per_cu(c->cfg.fmt_k, c->cfg.fmt_v, c->geom.group);
    if (cus <= 0 || per_cu <= 0) return KV_EDEVICE;
    const int64_t slots = (int64_t)cus * per_cu;
    int64_t min_wgs = 0;
    for (int i = 0; i < n_seqs; ++i)
        min_wgs += (int64_t)H * ((a.seqs[i].units_q > 0) + (a.seqs[i].units_t > 0));
    const int64_t waves = std::min<int64_t>(4, std::max<int64_t>(1, (8 * min_wgs + slots - 1) / slots));
    const int64_t target = std::min<int64_t>(slots * waves, max_wgs);
    auto plan = [&](int64_t uq, int64_t ut) {
        int64_t w = 0;
        for (int i = 0; i < n_seqs; ++i) {
            DecodeSeq& s = a.seqs[i];
            // quantized and ring units never share a workgroup: KVarN accumulates the
            // quantized values in the rotated domain, the ring values in the original one
            s.splits_q = (int32_t)((s.units_q + uq - 1) / uq);
            s.splits_t = (int32_t)((s.units_t + ut - 1) / ut);
            s.wg_base = (int32_t)w;
            w += (int64_t)H * (s.splits_q + s.splits_t);
        }
        return w;
    };
    auto t_lo = [](int64_t u) { return std::max<int64_t>(1, 4 * u / 5); };
    auto t_hi = [](int64_t u) { return std::max<int64_t>(1, (9 * u + 9) / 10); };
    // the fewest units per workgroup that fit the target (the count falls as units grow)
    int64_t lo = std::max<int64_t>(1, (total_units + 4 * target - 1) / (4 * target));
    int64_t hi = std::max<int64_t>(lo, std::max<int64_t>(max_uq, (10 * max_ut + 8) / 9 + 1));
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (plan(mid, t_hi(mid)) <= target) hi = mid; else lo = mid + 1;
    }
    const int64_t upw = lo;
    int64_t upw_t = t_hi(upw);
    for (int64_t t = t_lo(upw); t < t_hi(upw); ++t)
        if (plan(upw, t) <= target) { upw_t = t; break; }
    const int64_t wgs = plan(upw, upw_t);
    if (wgs > max_wgs) return KV_EUNSUPPORTED;
    a.units_per_wg = (int32_t)upw;
    a.units_per_wg_t = (int32_t)upw_t;
    int32_t qb = 0, tb = 0;
    for (int i = 0; i < n_seqs; ++i) {
        a.seqs[i].q_base = qb;
        a.seqs[i].t_base = tb;
        qb += H * a.seqs[i].splits_q;
        tb += H * a.seqs[i].splits_t;
    }
    a.q_wgs = qb;
    if (log_level() >= 2)
        std::fprintf(stderr,
                     "kvq: decode layer %d, %d sequences: %lld workgroups (%d quantized, %lld ring; %lld waves), "
                     "%lld pages or %lld ring units per workgroup\n",
                     layer, n_seqs, (long long)wgs, qb, (long long)(wgs - qb), (long long)waves, (long long)upw,
                     (long long)upw_t);
    int rc = launch_decode(a, (int)wgs, stream);
    return rc ? KV_EDEVICE : KV_OK;
}

}  // namespace

extern "C" {

int kv_decode_attn(kv_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                   const void* q, int32_t q_dtype, float softmax_scale, float* out,
                   void* workspace, int64_t ws_bytes, void* stream)
{
    int rc = decode_check(c, layer, n_seqs, seq_ids, q, q_dtype, softmax_scale, out);
    if (rc) return rc;
    if (!workspace) return KV_EINVAL;
    if (ws_bytes < kv_decode_workspace_bytes(c, n_seqs)) return KV_ESIZE;
    if ((rc = decode_nonempty(c, layer, n_seqs, seq_ids))) return rc;
    return decode_launch(c, layer, n_seqs, seq_ids, q, q_dtype, softmax_scale, out, workspace, kMaxDecodeWGs,
                         stream);
}

int kv_decode_attn_noalloc(kv_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                           const void* q, int32_t q_dtype, float softmax_scale, float* out, void* stream)
{
    int rc = decode_check(c, layer, n_seqs, seq_ids, q, q_dtype, softmax_scale, out);
    if (rc) return rc;
    if ((rc = decode_nonempty(c, layer, n_seqs, seq_ids))) return rc;
    // the smallest plan (one quantized and one ring split per sequence and KV head) must fit
    // the device array: a clear error before any device call
    if ((int64_t)n_seqs * c->cfg.n_kv_heads * 2 > kScratchWGs) return KV_ESIZE;
    int64_t bytes = 0;
    void* scratch = decode_scratch(&bytes);
    if (!scratch) return KV_EDEVICE;
    if (bytes < kScratchWGs * kPartialFloats * 4) return KV_EDEVICE;
    rc = decode_launch(c, layer, n_seqs, seq_ids, q, q_dtype, softmax_scale, out, scratch, kScratchWGs, stream);
    return rc == KV_EUNSUPPORTED ? KV_ESIZE : rc;
}

int kv_seq_get(const kv_cache* c, int32_t seq, int32_t layer, int64_t* n, int64_t* n_q)
{
    if (!c || seq < 0 || seq >= c->cfg.n_seqs || layer < 0 || layer >= c->cfg.n_layers) return KV_EINVAL;
    size_t i = (size_t)seq * c->cfg.n_layers + layer;
    if (n) *n = c->n[i];
    if (n_q) *n_q = c->nq[i];
    return KV_OK;
}

int kv_seq_set(kv_cache* c, int32_t seq, int32_t layer, int64_t n, int64_t n_q)
{
    if (!c || seq < 0 || seq >= c->cfg.n_seqs || layer < -1 || layer >= c->cfg.n_layers) return KV_EINVAL;
    if (n_q < 0 || n_q > n || n > c->cfg.max_tokens) return KV_EINVAL;
    if (n_q % c->granule) return KV_EINVAL;
    if (n - n_q > c->ring_slots) return KV_EINVAL;
    int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->cfg.n_layers : layer + 1;
    for (int l = l0; l < l1; ++l) {
        n_at(c, seq, l) = n;
        nq_at(c, seq, l) = n_q;
    }
    return KV_OK;
}

int kv_stream_layout(const kv_cache* c, int32_t seq, int32_t layer, int32_t kv_head, int32_t is_v,
                     int64_t offsets[4], int64_t* ring_slots)
{
    if (!c || !offsets || seq < 0 || seq >= c->cfg.n_seqs || layer < 0 || layer >= c->cfg.n_layers ||
        kv_head < 0 || kv_head >= c->cfg.n_kv_heads || (is_v != 0 && is_v != 1))
        return KV_EINVAL;
    int64_t unit = ((int64_t)seq * c->cfg.n_layers + layer) * c->cfg.n_kv_heads + kv_head;
    int64_t base = unit * c->geom.unit_bytes + (is_v ? c->geom.v_offset : 0);
    const StreamLayout& s = is_v ? c->geom.v : c->geom.k;
    offsets[0] = base + s.codes;
    offsets[1] = base + s.scales;
    offsets[2] = s.cscale < 0 ? -1 : base + s.cscale;
    offsets[3] = base + s.ring;
    if (ring_slots) *ring_slots = c->ring_slots;
    return KV_OK;
}

}  // extern "C"
