// kvq_decode_ws_k8.hip -- the fast decode kernel for 8-bit keys (q8_0, q8_1, kvarn8) against every
// value format of the fast kernel; one translation unit per key width so the builds run in
// parallel.
#include "kvq_decode_ws.h"

namespace kvq {

// op 0: launch (returns the HIP error), 1: workgroups per CU
int decode_fast_w8(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    switch (fmt_k) {
    case 11: return ws_value_switch<11>(op, fmt_v, a, n_wgs, st);
    case 12: return ws_value_switch<12>(op, fmt_v, a, n_wgs, st);
    case 18: return ws_value_switch<18>(op, fmt_v, a, n_wgs, st);
    default: return op == 0 ? (int)hipErrorInvalidValue : 0;
    }
}

}  // namespace kvq
