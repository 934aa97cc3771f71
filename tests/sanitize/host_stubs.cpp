// Host-only stand-ins for the device layer of the C-ABI library, for the sanitizer build
// of its host code (kvq_host.cpp).  No kernel runs: each launch checks the arguments the
// host code built (the decode split plan, the append entries) and returns success.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kvq_internal.h"

namespace kvq {

static void fail(const char* what)
{
    std::fprintf(stderr, "stub check failed: %s\n", what);
    std::abort();
}

int device_cu_count() { return 256; }
int decode_wgs_per_cu(int, int, int) { return 1; }

static float g_scratch[kScratchWGs * kPartialFloats];
void* decode_scratch(int64_t* bytes)
{
    *bytes = (int64_t)sizeof(g_scratch);
    return g_scratch;
}

// The plan covers every unit of every (sequence, KV head) exactly once, each split has at
// least one unit, and workgroup b -> split is a bijection onto the partial slots.
int launch_decode(const DecodeArgs& a, int n_wgs, void*)
{
    const int H = a.g.n_kv_heads;
    if (n_wgs < 1 || a.units_per_wg < 1 || a.units_per_wg_t < 1) fail("plan sizes");
    int64_t slots = 0, qw = 0, tw = 0;
    for (int i = 0; i < a.n_seqs; ++i) {
        const DecodeSeq& s = a.seqs[i];
        if (s.wg_base != slots || s.q_base != qw || s.t_base != tw) fail("plan bases");
        if ((int64_t)s.splits_q * a.units_per_wg < s.units_q ||
            (s.splits_q > 0 && (int64_t)(s.splits_q - 1) * a.units_per_wg >= s.units_q)) fail("quantized splits");
        if ((int64_t)s.splits_t * a.units_per_wg_t < s.units_t ||
            (s.splits_t > 0 && (int64_t)(s.splits_t - 1) * a.units_per_wg_t >= s.units_t)) fail("ring splits");
        if (s.units_q * 128 < s.n_q || s.units_t * 32 < s.n - s.n_q) fail("units");
        slots += (int64_t)H * (s.splits_q + s.splits_t);
        qw += (int64_t)H * s.splits_q;
        tw += (int64_t)H * s.splits_t;
    }
    if (slots != n_wgs || qw != a.q_wgs || qw + tw != n_wgs) fail("plan totals");
    // the same mapping the kernels use, on the host
    std::vector<int> seen((size_t)n_wgs, 0);
    for (int b = 0; b < n_wgs; ++b) {
        const bool quant = b < a.q_wgs;
        const int r0 = quant ? b : b - a.q_wgs;
        int e = 0;
        for (int i = 1; i < a.n_seqs; ++i)
            if ((quant ? a.seqs[i].q_base : a.seqs[i].t_base) <= r0) e = i;
        const DecodeSeq& s = a.seqs[e];
        const int rr = r0 - (quant ? s.q_base : s.t_base);
        const int ns = quant ? s.splits_q : s.splits_t;
        if (ns <= 0 || rr < 0 || rr >= H * ns) fail("workgroup mapping");
        const int head = rr / ns, sp = (quant ? 0 : s.splits_q) + rr % ns;
        const int slot = s.wg_base + head * (s.splits_q + s.splits_t) + sp;
        if (slot < 0 || slot >= n_wgs || seen[(size_t)slot]++) fail("partial slots");
    }
    return 0;
}

int launch_append_encode(const AppendArgs& a, void*)
{
    for (int i = 0; i < a.n_seqs; ++i)
        if (a.seqs[i].nq_new < a.seqs[i].nq_old) fail("append encode range");
    return 0;
}
int launch_append_kvarn(const AppendArgs& a, void*)
{
    for (int i = 0; i < a.n_seqs; ++i)
        if ((a.seqs[i].nq_new - a.seqs[i].nq_old) % 128) fail("kvarn page range");
    return 0;
}
int launch_append_ring(const AppendArgs&, void*) { return 0; }
int launch_prefill(const PrefillArgs&, void*) { return 0; }
int launch_kld(const KldArgs&, void*) { return 0; }

}  // namespace kvq
