// kvq_decode_ws.hip -- dispatch of the fast decode kernel (kvq_decode_ws.h) by key width.
#include "kvq_device.h"

namespace kvq {

int decode_fast_w2(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream);
int decode_fast_w3(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream);
int decode_fast_w4(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream);
int decode_fast_w5(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream);
int decode_fast_w6(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream);
int decode_fast_w8(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream);

namespace {

// formats of the fast kernel: qN_0, qN_1 and kvarnN (kvarnN_1 and bf16 take the generic kernel)
bool fast_format(int f)
{
    return f >= 1 && f < kNumFormats && (fkind(f) == KIND_Q0 || fkind(f) == KIND_Q1 || fkind(f) == KIND_KVARN);
}

int by_width(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream)
{
    switch (fbits(fmt_k)) {
    case 2: return decode_fast_w2(op, a, fmt_k, fmt_v, n_wgs, stream);
    case 3: return decode_fast_w3(op, a, fmt_k, fmt_v, n_wgs, stream);
    case 4: return decode_fast_w4(op, a, fmt_k, fmt_v, n_wgs, stream);
    case 5: return decode_fast_w5(op, a, fmt_k, fmt_v, n_wgs, stream);
    case 6: return decode_fast_w6(op, a, fmt_k, fmt_v, n_wgs, stream);
    case 8: return decode_fast_w8(op, a, fmt_k, fmt_v, n_wgs, stream);
    default: return op == 0 ? (int)hipErrorInvalidValue : 0;
    }
}

}  // namespace

bool decode_fast_supported(int fmt_k, int fmt_v)
{
    return fast_format(fmt_k) && fast_format(fmt_v);
}

int launch_decode_fast(const DecodeArgs& a, int n_wgs, void* stream)
{
    if (!decode_fast_supported(a.g.fmt_k, a.g.fmt_v)) return (int)hipErrorInvalidValue;
    return by_width(0, &a, a.g.fmt_k, a.g.fmt_v, n_wgs, stream);
}

int decode_fast_wgs_per_cu(int fmt_k, int fmt_v)
{
    static int cache[kNumFormats][kNumFormats] = {{0}};
    if (!decode_fast_supported(fmt_k, fmt_v)) return 0;
    if (!cache[fmt_k][fmt_v]) cache[fmt_k][fmt_v] = by_width(1, nullptr, fmt_k, fmt_v, 0, nullptr);
    return cache[fmt_k][fmt_v];
}

}  // namespace kvq
