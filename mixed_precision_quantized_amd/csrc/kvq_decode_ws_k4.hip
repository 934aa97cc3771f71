// kvq_decode_ws_k4.hip -- the fast decode kernel for 4-bit keys (q4_0, q4_1, kvarn4) against every
// value format of the fast kernel; one translation unit per key width so the builds run in
// parallel.
#include "kvq_decode_ws.h"

namespace kvq {

// op 0: launch (returns the HIP error), 1: workgroups per CU
int decode_fast_w4(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    switch (fmt_k) {
    case 5: return ws_value_switch<5>(op, fmt_v, a, n_wgs, st);
    case 6: return ws_value_switch<6>(op, fmt_v, a, n_wgs, st);
    case 15: return ws_value_switch<15>(op, fmt_v, a, n_wgs, st);
    default: return op == 0 ? (int)hipErrorInvalidValue : 0;
    }
}

}  // namespace kvq
