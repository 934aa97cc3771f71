// kvq_merge.hip -- combine the split-K partial results of decode attention, gfx950.
//
// Each decode workgroup leaves, per query head of its KV head, the running maximum m, the
// normalizer l and the unnormalized accumulator acc[128] of its share of the tokens (log2
// domain: p_t = 2^(s_t - m)).  This kernel, launched after the decode kernel on the same
// stream, merges them (flash-decoding reduction):
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  O = sum_s acc_s 2^(m_s - M) / L.
// A separate launch instead of a last-workgroup merge inside the decode kernel: the kernel
// boundary publishes the partials, where an in-kernel handoff would need a device-scope
// release fence in every workgroup, and each such fence writes back the whole L2 of its
// XCD while the other workgroups are still streaming the cache.
//
// KVarN: the quantized splits accumulate rotated values (Yhat, with x = H Yhat / 128 and H
// the unnormalized Sylvester Hadamard matrix), the BF16 ring splits original values; the
// quantized sum is rotated back here once, before the two are added.
#include "kvq_device.h"

namespace kvq {

namespace {

constexpr int kG = 4;
constexpr int kCols = kD / 4;                 // float4 columns of one head's accumulator
constexpr int kGroups = 256 / kCols;          // split groups in the accumulation phase

// One workgroup per (sequence, KV head, query head of the group).
template <bool KVARN>
__global__ __launch_bounds__(256) void k_merge(DecodeArgs a)
{
    __shared__ float4 red[kGroups][2][kCols];  // [split group][quantized | ring][column]
    __shared__ float vq[kD], vt[kD];
    __shared__ float wm[4], wl[4];
    __shared__ float ML[2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.g.n_kv_heads;
    const int e = blockIdx.x / (H * kG);
    const int head = (blockIdx.x / kG) % H;
    const int h = blockIdx.x % kG;
    const DecodeSeq& sq = a.seqs[e];
    const int SPL = sq.splits_q + sq.splits_t;
    const float* parts = a.partials + (int64_t)(sq.wg_base + head * SPL) * kPartialFloats;

    // maximum and normalizer: one online pass per thread, then across the workgroup
    float mx = -1.0e30f, L = 0.0f;
    for (int s = tid; s < SPL; s += 256) {
        const float m = parts[(int64_t)s * kPartialFloats + h];
        const float l = parts[(int64_t)s * kPartialFloats + kMaxGroup + h];
        const float nm = fmaxf(mx, m);
        L = L * __builtin_amdgcn_exp2f(mx - nm) + l * __builtin_amdgcn_exp2f(m - nm);
        mx = nm;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float m2 = __shfl_xor(mx, o), l2 = __shfl_xor(L, o);
        const float nm = fmaxf(mx, m2);
        L = L * __builtin_amdgcn_exp2f(mx - nm) + l2 * __builtin_amdgcn_exp2f(m2 - nm);
        mx = nm;
    }
    if (lane == 0) { wm[wave] = mx; wl[wave] = L; }
    __syncthreads();
    if (tid == 0) {
        float M = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
        float T = 0.0f;
        for (int w = 0; w < 4; ++w) T += wl[w] * __builtin_amdgcn_exp2f(wm[w] - M);
        ML[0] = M;
        ML[1] = T;
    }
    __syncthreads();
    const float M = ML[0];

    // rescaled accumulators: thread = (split group, float4 column)
    {
        const int c = tid % kCols, sg = tid / kCols;
        float4 aq = make_float4(0.0f, 0.0f, 0.0f, 0.0f), at = aq;
#pragma unroll 4
        for (int s = sg; s < SPL; s += kGroups) {
            const float* pp = parts + (int64_t)s * kPartialFloats;
            const float w = __builtin_amdgcn_exp2f(pp[h] - M);
            const float4 v = *(const float4*)(pp + 2 * kMaxGroup + h * kD + 4 * c);
            float4& d = s < sq.splits_q ? aq : at;
            d.x = fmaf(v.x, w, d.x);
            d.y = fmaf(v.y, w, d.y);
            d.z = fmaf(v.z, w, d.z);
            d.w = fmaf(v.w, w, d.w);
        }
        red[sg][0][c] = aq;
        red[sg][1][c] = at;
    }
    __syncthreads();
    if (tid < kD) {
        const int c = tid >> 2, k = tid & 3;
        float sq_ = 0.0f, st = 0.0f;
        for (int g = 0; g < kGroups; ++g) {
            sq_ += reinterpret_cast<const float*>(&red[g][0][c])[k];
            st += reinterpret_cast<const float*>(&red[g][1][c])[k];
        }
        vq[tid] = sq_;
        vt[tid] = st;
    }
    if (KVARN) {
        // x = H yhat / 128, butterflies of span 1, 2, .., 64
        for (int span = 1; span < kD; span <<= 1) {
            __syncthreads();
            if (tid < kD / 2) {
                const int lo = tid & (span - 1);
                const int i = ((tid - lo) << 1) | lo;
                const float x = vq[i], y = vq[i + span];
                vq[i] = x + y;
                vq[i + span] = x - y;
            }
        }
    }
    __syncthreads();
    if (tid < kD) {
        float q = vq[tid];
        if (KVARN) q *= (1.0f / 128.0f);
        a.out[((int64_t)sq.in_idx * a.g.n_q_heads + head * kG + h) * kD + tid] = (q + vt[tid]) / ML[1];
    }
}

}  // namespace

int launch_merge(const DecodeArgs& a, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    const int n = a.n_seqs * a.g.n_kv_heads * kG;
    if (fkind(a.g.fmt_k) == KIND_KVARN)
        hipLaunchKernelGGL(k_merge<true>, dim3(n), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(k_merge<false>, dim3(n), dim3(256), 0, st, a);
    return (int)hipGetLastError();
}

}  // namespace kvq
