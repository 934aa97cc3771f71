// kvq_decode_ws_k5.hip -- the fast decode kernel for 5-bit keys (q5_0, q5_1, kvarn5) against every
// value format of the fast kernel; one translation unit per key width so the builds run in
// parallel.
#include "kvq_decode_ws.h"

namespace kvq {

// op 0: launch (returns the HIP error), 1: workgroups per CU
int decode_fast_w5(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    switch (fmt_k) {
    case 7: return ws_value_switch<7>(op, fmt_v, a, n_wgs, st);
    case 8: return ws_value_switch<8>(op, fmt_v, a, n_wgs, st);
    case 16: return ws_value_switch<16>(op, fmt_v, a, n_wgs, st);
    default: return op == 0 ? (int)hipErrorInvalidValue : 0;
    }
}

}  // namespace kvq
