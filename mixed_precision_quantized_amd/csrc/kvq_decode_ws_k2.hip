// kvq_decode_ws_k2.hip -- the fast decode kernel for 2-bit keys (q2_0, q2_1, kvarn2) against every
// value format of the fast kernel; one translation unit per key width so the builds run in
// parallel.
#include "kvq_decode_ws.h"

namespace kvq {

// op 0: launch (returns the HIP error), 1: workgroups per CU
int decode_fast_w2(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    switch (fmt_k) {
    case 1: return ws_value_switch<1>(op, fmt_v, a, n_wgs, st);
    case 2: return ws_value_switch<2>(op, fmt_v, a, n_wgs, st);
    case 13: return ws_value_switch<13>(op, fmt_v, a, n_wgs, st);
    default: return op == 0 ? (int)hipErrorInvalidValue : 0;
    }
}

}  // namespace kvq
