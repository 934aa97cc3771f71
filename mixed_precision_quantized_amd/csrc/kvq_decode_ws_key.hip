// kvq_decode_ws_key.hip -- the fast decode kernel for one key format against every value
// format.  The key format id comes from the command line (-DKVQ_WS_FK=<id>): the file is
// compiled once per key format, so the 24 x 24 instantiations build in parallel.
#include "kvq_decode_ws.h"

#ifndef KVQ_WS_FK
#error "KVQ_WS_FK (the key format id, 1..24) must be defined"
#endif

namespace kvq {

// op 0: launch (returns the HIP error), 1: workgroups per CU
template <int FK>
int decode_fast_key(int op, const DecodeArgs* a, int fmt_v, int n_wgs, void* stream)
{
    return ws_value_switch<FK>(op, fmt_v, a, n_wgs, (hipStream_t)stream);
}

template int decode_fast_key<KVQ_WS_FK>(int, const DecodeArgs*, int, int, void*);

}  // namespace kvq
