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
// KVarN (both inner quantizers): the quantized splits accumulate rotated values (Yhat, with x = H Yhat / 128 and H
// the unnormalized Sylvester Hadamard matrix), the BF16 ring splits original values; the
// quantized sum is rotated back here once, before the two are added.
#include <mutex>

#include "kvq_device.h"

namespace kvq {

// Split partials of kv_decode_attn_noalloc, for callers that cannot allocate: one array of
// kScratchWGs partials (4,259,840 bytes) per device, kept until the process ends and shared
// by every such call on that device.  The partials need no initialization (each workgroup
// writes its own in full).
static __device__ __align__(256) float scratch[kScratchWGs * kPartialFloats];

namespace {

constexpr int kG = 4;
constexpr int kCols = kD / 4;                 // float4 columns of one head's accumulator
constexpr int kGroups = 8;                    // split groups: thread = (group, column)
constexpr int kThreads = kGroups * kCols;     // 256

// One workgroup per (sequence, KV head, query head of the group).  Thread (g, c) folds
// float4 column c over the splits g, g + 8, ... with its own running maximum, all loads of
// a batch issued together; the 8 groups then combine through LDS (three barriers), and
// wave 0 finishes the dims in registers: lane l holds dims l and l + 64, so the inverse
// rotation of KVarN is one in-lane butterfly (span 64) and six cross-lane ones.
template <bool KVARN>
__global__ __launch_bounds__(kThreads) void k_merge(DecodeArgs a)
{
    __shared__ float4 rq[kGroups][kCols], rt[kGroups][kCols];   // [group][column]
    __shared__ float gm[kGroups], gl[kGroups];
    __shared__ float vq[kD], vt[kD];

    const int tid = threadIdx.x, c = tid % kCols, g = tid / kCols;
    const int H = a.g.n_kv_heads;
    const int e = blockIdx.x / (H * kG);
    const int head = (blockIdx.x / kG) % H;
    const int h = blockIdx.x % kG;
    const DecodeSeq& sq = a.seqs[e];
    const int SPL = sq.splits_q + sq.splits_t;
    const float* parts = a.partials + (int64_t)(sq.wg_base + head * SPL) * kPartialFloats;

    float mx = -1.0e30f, L = 0.0f;
    float4 aq = make_float4(0.0f, 0.0f, 0.0f, 0.0f), at = aq;
    // batches of kBatch splits per thread: all loads of a batch are issued before any is used
    // (indices clamped to the last split, the surplus is masked out)
    constexpr int kBatch = 4;
    for (int s0 = g; s0 < SPL; s0 += kBatch * kGroups) {
        float m[kBatch], l[kBatch];
        float4 v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const float* pp = parts + (int64_t)min(s0 + i * kGroups, SPL - 1) * kPartialFloats;
            m[i] = pp[h];
            l[i] = pp[kMaxGroup + h];
            v[i] = *(const float4*)(pp + 2 * kMaxGroup + h * kD + 4 * c);
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int s = s0 + i * kGroups;
            if (s >= SPL) break;
            const float nm = fmaxf(mx, m[i]);
            const float r = __builtin_amdgcn_exp2f(mx - nm), w = __builtin_amdgcn_exp2f(m[i] - nm);
            mx = nm;
            L = fmaf(L, r, l[i] * w);
            const bool isq = s < sq.splits_q;
            const float4 x = v[i];
            aq.x = fmaf(aq.x, r, isq ? x.x * w : 0.0f); aq.y = fmaf(aq.y, r, isq ? x.y * w : 0.0f);
            aq.z = fmaf(aq.z, r, isq ? x.z * w : 0.0f); aq.w = fmaf(aq.w, r, isq ? x.w * w : 0.0f);
            at.x = fmaf(at.x, r, isq ? 0.0f : x.x * w); at.y = fmaf(at.y, r, isq ? 0.0f : x.y * w);
            at.z = fmaf(at.z, r, isq ? 0.0f : x.z * w); at.w = fmaf(at.w, r, isq ? 0.0f : x.w * w);
        }
    }
    if (c == 0) { gm[g] = mx; gl[g] = L; }
    __syncthreads();
    // every thread: the common maximum and the normalizer over the 8 groups
    float M = gm[0];
#pragma unroll
    for (int gg = 1; gg < kGroups; ++gg) M = fmaxf(M, gm[gg]);
    float T = 0.0f;
#pragma unroll
    for (int gg = 0; gg < kGroups; ++gg) T += gl[gg] * __builtin_amdgcn_exp2f(gm[gg] - M);
    {
        // rescale to the common maximum before the sum, so the column sums below are plain adds
        const float w = __builtin_amdgcn_exp2f(mx - M);
        rq[g][c] = make_float4(aq.x * w, aq.y * w, aq.z * w, aq.w * w);
        rt[g][c] = make_float4(at.x * w, at.y * w, at.z * w, at.w * w);
    }
    __syncthreads();
    {
        // thread = (quantized | ring part, dim): 8 adds down the groups
        const int part = tid / kD, d = tid % kD, cc = d >> 2, k = d & 3;
        const float4 (*r)[kCols] = part ? rt : rq;
        float sum = 0.0f;
#pragma unroll
        for (int gg = 0; gg < kGroups; ++gg) sum += reinterpret_cast<const float*>(&r[gg][cc])[k];
        (part ? vt : vq)[d] = sum;
    }
    __syncthreads();
    if (tid < 64) {
        const int l = tid;
        float x0 = vq[l], x1 = vq[l + 64];
        if (KVARN) {
            // x = H yhat / 128: span 64 inside the lane, spans 32 .. 1 across lanes
            const float u = x0 + x1, w = x0 - x1;
            x0 = u;
            x1 = w;
#pragma unroll
            for (int sp = 32; sp >= 1; sp >>= 1) {
                const float y0 = __shfl_xor(x0, sp), y1 = __shfl_xor(x1, sp);
                const bool up = (l & sp) != 0;
                x0 = up ? y0 - x0 : x0 + y0;
                x1 = up ? y1 - x1 : x1 + y1;
            }
            x0 *= (1.0f / 128.0f);
            x1 *= (1.0f / 128.0f);
        }
        float* o = a.out + ((int64_t)sq.in_idx * a.g.n_q_heads + head * kG + h) * kD;
        o[l] = (x0 + vt[l]) / T;
        o[l + 64] = (x1 + vt[l + 64]) / T;
    }
}

}  // namespace

// Device address of this device's `scratch`, looked up on the first call per device with
// that device current (the host-side name is not a device address).
void* decode_scratch(int64_t* bytes)
{
    constexpr int kMaxDevices = 64;
    static void* ptr[kMaxDevices] = {nullptr};
    static std::mutex mu;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        ptr[dev] = p;
    }
    *bytes = (int64_t)sizeof(scratch);
    return ptr[dev];
}

int launch_merge(const DecodeArgs& a, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    const int n = a.n_seqs * a.g.n_kv_heads * kG;
    if (kind_paged(fkind(a.g.fmt_v)))        // values accumulated in the rotated domain
        hipLaunchKernelGGL(k_merge<true>, dim3(n), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(k_merge<false>, dim3(n), dim3(kThreads), 0, st, a);
    return (int)hipGetLastError();
}

}  // namespace kvq
