// kvq_decode_ws.hip -- dispatch of the fast decode kernel (kvq_decode_ws.h) by key format.
#include "kvq_device.h"

namespace kvq {

// defined in kvq_decode_ws_key.hip, one translation unit per key format
template <int FK>
int decode_fast_key(int op, const DecodeArgs* a, int fmt_v, int n_wgs, void* stream);

namespace {

// formats of the fast kernel: every quantized format (qN_0, qN_1, kvarnN, kvarnN_1)
bool fast_format(int f)
{
    return f >= 1 && f < kNumFormats && fkind(f) != KIND_BF16;
}

int by_key(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream)
{
#define KVQ_WS_KEY(F) \
    case F: return decode_fast_key<F>(op, a, fmt_v, n_wgs, stream);
    switch (fmt_k) {
        KVQ_WS_KEY(1) KVQ_WS_KEY(2) KVQ_WS_KEY(3) KVQ_WS_KEY(4) KVQ_WS_KEY(5) KVQ_WS_KEY(6)
        KVQ_WS_KEY(7) KVQ_WS_KEY(8) KVQ_WS_KEY(9) KVQ_WS_KEY(10) KVQ_WS_KEY(11) KVQ_WS_KEY(12)
        KVQ_WS_KEY(13) KVQ_WS_KEY(14) KVQ_WS_KEY(15) KVQ_WS_KEY(16) KVQ_WS_KEY(17) KVQ_WS_KEY(18)
        KVQ_WS_KEY(19) KVQ_WS_KEY(20) KVQ_WS_KEY(21) KVQ_WS_KEY(22) KVQ_WS_KEY(23) KVQ_WS_KEY(24)
    default: return op == 0 ? (int)hipErrorInvalidValue : 0;
    }
#undef KVQ_WS_KEY
}

}  // namespace

bool decode_fast_supported(int fmt_k, int fmt_v)
{
    return fast_format(fmt_k) && fast_format(fmt_v);
}

int launch_decode_fast(const DecodeArgs& a, int n_wgs, void* stream)
{
    if (!decode_fast_supported(a.g.fmt_k, a.g.fmt_v)) return (int)hipErrorInvalidValue;
    return by_key(0, &a, a.g.fmt_k, a.g.fmt_v, n_wgs, stream);
}

int decode_fast_wgs_per_cu(int fmt_k, int fmt_v)
{
    static int cache[kNumFormats][kNumFormats] = {{0}};
    if (!decode_fast_supported(fmt_k, fmt_v)) return 0;
    if (!cache[fmt_k][fmt_v]) cache[fmt_k][fmt_v] = by_key(1, nullptr, fmt_k, fmt_v, 0, nullptr);
    return cache[fmt_k][fmt_v];
}

}  // namespace kvq
