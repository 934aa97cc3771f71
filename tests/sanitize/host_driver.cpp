// Drives the C-ABI's host code through the sanitizer build (device layer stubbed): cache
// sizing and creation for every format pair and tail type, appends of ragged chunks with
// spills, every decode plan over 1..32 sequences of random lengths, the no-alloc entry
// point, prefill / KL workspace sizing, sequence state and stream layout, and the error
// paths of each call.  Prints "ok" and exits 0 when every call returns what it should.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kvq.h"

static int g_fail = 0;
#define EXPECT(c) do { if (!(c)) { std::fprintf(stderr, "line %d: %s\n", __LINE__, #c); g_fail = 1; } } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint64_t next()
{
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return rng;
}

static kv_config config(int L, int H, int fk, int fv, int T, int S, int64_t maxt, int tail_dtype)
{
    kv_config c{};
    c.n_layers = L; c.n_kv_heads = H; c.n_q_heads = 4 * H; c.head_dim = 128;
    c.fmt_k = fk; c.fmt_v = fv; c.tail_tokens = T; c.n_seqs = S; c.max_tokens = maxt;
    c.tail_dtype = tail_dtype;
    return c;
}

int main()
{
    // sizing and creation: every format pair, both tail types
    for (int fk = 0; fk < KV_NUM_FORMATS; ++fk)
        for (int fv = 0; fv < KV_NUM_FORMATS; fv += 5) {
            kv_config c = config(2, 2, fk, fv, 64, 2, 1000, (fk + fv) & 1);
            const int64_t b = kv_cache_bytes(&c);
            if (c.tail_dtype == KV_TAIL_F16 && (fk == KV_BF16 || fv == KV_BF16)) {
                EXPECT(b == KV_EUNSUPPORTED);       // an F16 tail holds no BF16 stream
                continue;
            }
            EXPECT(b > 0);
            std::vector<char> mem((size_t)b + 256);
            char* p = (char*)(((uintptr_t)mem.data() + 255) & ~(uintptr_t)255);
            kv_cache* h = nullptr;
            EXPECT(kv_cache_init(&c, p, b, &h) == KV_OK && h);
            kv_cache* h2 = nullptr;
            EXPECT(kv_cache_init(&c, p, b - 1, &h2) != KV_OK);
            kv_cache_destroy(h);
        }
    // bad configurations
    {
        kv_config c = config(1, 1, 5, 5, 16, 1, 100, 0);
        c.head_dim = 64; EXPECT(kv_cache_bytes(&c) < 0);
        c = config(1, 1, 5, 5, 16, 1, 100, 0); c.n_q_heads = 8; EXPECT(kv_cache_bytes(&c) == KV_EUNSUPPORTED);
        c = config(0, 1, 5, 5, 16, 1, 100, 0); EXPECT(kv_cache_bytes(&c) < 0);
        c = config(1, 1, 99, 5, 16, 1, 100, 0); EXPECT(kv_cache_bytes(&c) < 0);
        EXPECT(kv_cache_bytes(nullptr) < 0);
    }
    // large appends: every layer at once, then one layer at a time (over a million
    // token-heads per call), bf16 and f32 input
    for (int fk : {14, 5}) {
        const int L = 8, H = 8, S = 32, T = 1024;
        kv_config c = config(L, H, fk, fk, T, S, 20000, 0);
        const int64_t b = kv_cache_bytes(&c);
        EXPECT(b > 0);
        std::vector<char> mem(4096);
        char* p = (char*)(((uintptr_t)mem.data() + 255) & ~(uintptr_t)255);
        kv_cache* h = nullptr;
        EXPECT(kv_cache_init(&c, p, b, &h) == KV_OK);
        std::vector<int32_t> ids(S), nn(S, 4096);
        for (int s = 0; s < S; ++s) ids[s] = s;
        EXPECT(kv_append(h, -1, S, ids.data(), nn.data(), (void*)16, (void*)16, KV_IN_BF16, nullptr) == KV_OK);
        for (int l = 0; l < L; ++l)
            EXPECT(kv_append(h, l, S, ids.data(), nn.data(), (void*)16, (void*)16, KV_IN_F32, nullptr) == KV_OK);
        for (int s = 0; s < S; ++s) {
            int64_t n = -1, nq = -1;
            EXPECT(kv_seq_get(h, s, L - 1, &n, &nq) == KV_OK);
            EXPECT(n == 8192 && n - nq <= T + 128 && n - nq >= T);
        }
        kv_cache_destroy(h);
    }
    // a cache of 32 sequences: appends, spills, decode plans
    const int fmts[][2] = {{15, 15}, {5, 5}, {14, 14}, {0, 0}, {11, 5}, {21, 21}};
    for (auto& fp : fmts) {
        const int L = 3, H = 8, S = 32, T = 256;
        const int64_t maxt = 6000;
        kv_config c = config(L, H, fp[0], fp[1], T, S, maxt, 0);
        const int64_t b = kv_cache_bytes(&c);
        EXPECT(b > 0);
        // the device buffer is never touched by the host code: a small host block stands in
        std::vector<char> mem(4096);
        char* p = (char*)(((uintptr_t)mem.data() + 255) & ~(uintptr_t)255);
        kv_cache* h = nullptr;
        EXPECT(kv_cache_init(&c, p, b, &h) == KV_OK);
        std::vector<int32_t> ids(S), nn(S);
        for (int s = 0; s < S; ++s) ids[s] = s;
        std::vector<int64_t> len(S, 0);
        for (int round = 0; round < 6; ++round) {
            int64_t tot = 0;
            for (int s = 0; s < S; ++s) {
                nn[s] = (int32_t)(next() % 900);
                if (len[s] + nn[s] > maxt) nn[s] = (int32_t)(maxt - len[s]);
                tot += nn[s];
            }
            const int layer = round % 2 ? -1 : (int)(next() % L);
            EXPECT(kv_append(h, layer, S, ids.data(), nn.data(), (void*)16, (void*)16, KV_IN_BF16, nullptr) == KV_OK);
            if (layer == -1)
                for (int s = 0; s < S; ++s) len[s] += nn[s];
            else
                for (int s = 0; s < S; ++s) { (void)tot; }
            if (layer != -1) {
                // keep every layer at the same length: append the same chunk to the others
                for (int l = 0; l < L; ++l)
                    if (l != layer)
                        EXPECT(kv_append(h, l, S, ids.data(), nn.data(), (void*)16, (void*)16, KV_IN_BF16, nullptr) == KV_OK);
                for (int s = 0; s < S; ++s) len[s] += nn[s];
            }
            for (int s = 0; s < S; ++s) {
                int64_t n = -1, nq = -1;
                EXPECT(kv_seq_get(h, s, 0, &n, &nq) == KV_OK);
                EXPECT(n == len[s] && nq <= n && n - nq <= T + 128);
            }
            // decode over every prefix of the sequence list, and a random subset
            const int64_t ws = kv_decode_workspace_bytes(h, S);
            EXPECT(ws > 0);
            std::vector<int32_t> nz;
            for (int s = 0; s < S; ++s)
                if (len[s] > 0) nz.push_back(s);
            for (size_t k = 1; k <= nz.size(); k += 3) {
                EXPECT(kv_decode_attn(h, 0, (int32_t)k, nz.data(), (void*)16, KV_IN_BF16, 0.088f,
                                      (float*)16, (void*)16, ws, nullptr) == KV_OK);
                const int rc = kv_decode_attn_noalloc(h, 1, (int32_t)k, nz.data(), (void*)16, KV_IN_BF16, 0.088f,
                                                      (float*)16, nullptr);
                EXPECT(rc == KV_OK || rc == KV_ESIZE);
            }
            if (!nz.empty()) {
                EXPECT(kv_decode_attn(h, 0, 1, nz.data(), (void*)16, KV_IN_BF16, 0.088f, (float*)16, (void*)16, ws - 1,
                                      nullptr) == KV_ESIZE);
                const int32_t s0 = nz[0];
                EXPECT(kv_spill_tail(h, -1, s0, (int32_t)(next() % (T + 1)), nullptr) == KV_OK);
                const int64_t pw = kv_prefill_workspace_bytes(h, 1);
                EXPECT(pw > 0);
                EXPECT(kv_prefill_attn(h, 0, s0, 1, (void*)16, KV_IN_BF16, 0.088f, (float*)16, (void*)16, pw, nullptr) == KV_OK ||
                       fp[0] != fp[1]);
                const int64_t kw = kv_attn_kld_workspace_bytes(h);
                EXPECT(kw > 0);
            }
            // an empty sequence is an error for decode
            int32_t empty = -1;
            for (int s = 0; s < S; ++s)
                if (len[s] == 0) empty = s;
            if (empty >= 0)
                EXPECT(kv_decode_attn(h, 0, 1, &empty, (void*)16, KV_IN_BF16, 0.088f, (float*)16, (void*)16, ws, nullptr) ==
                       KV_EEMPTY);
        }
        // error paths
        EXPECT(kv_append(h, L, 1, ids.data(), nn.data(), (void*)16, (void*)16, KV_IN_BF16, nullptr) == KV_EINVAL);
        EXPECT(kv_append(h, 0, 1, nullptr, nn.data(), (void*)16, (void*)16, KV_IN_BF16, nullptr) == KV_EINVAL);
        int32_t big = (int32_t)maxt + 1;
        EXPECT(kv_append(h, 0, 1, ids.data(), &big, (void*)16, (void*)16, KV_IN_BF16, nullptr) != KV_OK);
        int32_t dup[2] = {1, 1}, one[2] = {1, 1};
        EXPECT(kv_append(h, 0, 2, dup, one, (void*)16, (void*)16, KV_IN_BF16, nullptr) == KV_EINVAL);
        EXPECT(kv_decode_attn(h, 0, 0, ids.data(), (void*)16, KV_IN_BF16, 0.088f, (float*)16, (void*)16, 1 << 30, nullptr) ==
               KV_EINVAL);
        EXPECT(kv_seq_get(h, S, 0, nullptr, nullptr) == KV_EINVAL);
        EXPECT(kv_seq_set(h, 0, 0, 10, 11) == KV_EINVAL);
        int64_t off[4], slots = 0;
        EXPECT(kv_stream_layout(h, 1, 2, 7, 1, off, &slots) == KV_OK && slots > 0);
        EXPECT(kv_stream_layout(h, 1, 2, 8, 1, off, &slots) == KV_EINVAL);
        // restore state to a clone (the host side of a checkpoint round trip)
        for (int s = 0; s < S; ++s) {
            int64_t n, nq;
            EXPECT(kv_seq_get(h, s, 0, &n, &nq) == KV_OK);
            EXPECT(kv_seq_set(h, s, -1, n, nq) == KV_OK);
        }
        EXPECT(kv_cache_destroy(h) == KV_OK);
    }
    EXPECT(kv_cache_destroy(nullptr) == KV_OK);
    int32_t bits, cb, sb, pb;
    for (int f = 0; f < KV_NUM_FORMATS; ++f) EXPECT(kv_format_info(f, &bits, &cb, &sb, &pb) == KV_OK);
    EXPECT(kv_format_info(KV_NUM_FORMATS, &bits, &cb, &sb, &pb) != KV_OK);
    if (g_fail) return 1;
    std::printf("ok\n");
    return 0;
}
