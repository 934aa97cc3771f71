// kvq_debug.hip -- device conversions exposed for exhaustive CPU comparison.
#pragma clang fp contract(off)

#include "kvq_debug.h"
#include "kvq_device.h"

namespace {

__global__ __launch_bounds__(256) void k_convert(const float* in, int64_t n, uint16_t* bo, uint16_t* ho,
                                                 float* ro, float* so)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float x = in[i];
    if (bo) bo[i] = kvq::bf16_rne(x);
    if (ho) ho[i] = kvq::fp16s_rne(x);
    if (ro) ro[i] = 1.0f / x;
    if (so) so[i] = __builtin_sqrtf(x);
}

}  // namespace

extern "C" int kv_debug_convert(const float* in, int64_t n, uint16_t* bf16_out, uint16_t* fp16_out,
                                float* recip_out, float* sqrt_out, void* stream)
{
    if (n < 0 || (!in && n > 0)) return -1;
    if (n == 0) return 0;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFF) return -1;
    hipLaunchKernelGGL(k_convert, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, in, n,
                       bf16_out, fp16_out, recip_out, sqrt_out);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int kv_debug_decode_events(void* before, void* after)
{
    return kvq::set_decode_events(before, after);
}
