// kvq_decode_ws_k3.hip -- the fast decode kernel for 3-bit keys (q3_0, q3_1, kvarn3) against every
// value format of the fast kernel; one translation unit per key width so the builds run in
// parallel.
#include "kvq_decode_ws.h"

namespace kvq {

// op 0: launch (returns the HIP error), 1: workgroups per CU
int decode_fast_w3(int op, const DecodeArgs* a, int fmt_k, int fmt_v, int n_wgs, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    switch (fmt_k) {
    case 3: return ws_value_switch<3>(op, fmt_v, a, n_wgs, st);
    case 4: return ws_value_switch<4>(op, fmt_v, a, n_wgs, st);
    case 14: return ws_value_switch<14>(op, fmt_v, a, n_wgs, st);
    default: return op == 0 ? (int)hipErrorInvalidValue : 0;
    }
}

}  // namespace kvq
