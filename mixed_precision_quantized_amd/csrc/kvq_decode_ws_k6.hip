// kvq_decode_ws_k6.hip -- the fast decode kernel for 6-bit keys (q6_0, q6_1, kvarn6) against every
// value format of the fast kernel; one translation unit per key width so the builds run in
// parallel.
#include "kvq_decode_ws.h"

namespace kvq {

// op 0: launch (returns the HIP error), 1: workgroups per CU
int decode_fast_w6(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    switch (fmt_k) {
    case 9: return ws_value_switch<9>(op, fmt_v, a, n_wgs, st);
    case 10: return ws_value_switch<10>(op, fmt_v, a, n_wgs, st);
    case 17: return ws_value_switch<17>(op, fmt_v, a, n_wgs, st);
    default: return op == 0 ? (int)hipErrorInvalidValue : 0;
    }
}

}  // namespace kvq
