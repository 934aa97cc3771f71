// kvq_decode.hip -- single-token GQA decode attention over the mixed-precision cache, gfx950.
//
// Long-context decode is a streaming read of the whole cache (memory bound: "Форк beellama
// и KV-кванты kvarn на длинном контексте: что известно об ускорении в 2026 году", section
// "Длинный контекст меняет профиль нагрузки с вычислений на работу с памятью"), so the
// kernel reads every packed row once, coalesced, and dequantizes in registers.  It is not
// a dense contraction at 4 query heads per KV head: no matrix cores.
//
// This binary32 kernel serves the pairs that hold a bf16 stream (bf16 keys, bf16 values or
// both); every pair of quantized formats runs the matrix-core kernel of kvq_decode_ws.h.
// Its dequantization also feeds the attention-KL harness at the end of this file.
//
// Work split (split-K flash decode): the tokens of each (sequence, KV head) are cut into
// units (128-token quantized pages, 32-token ring chunks); every workgroup owns a run of
// units of one kind, sized so the whole grid is resident at once.  Each wave keeps an
// online softmax (running max m, sum l, accumulator acc) per token slot; slots and waves
// merge through shuffles and LDS into one partial result per workgroup, and a second
// launch (kvq_merge.hip) merges the partials of each (sequence, KV head).
//
// KVarN: keys and values are stored rotated, x = H Yhat / 128 with H the unnormalized
// Sylvester Hadamard matrix (symmetric).  So q.x = (H q / 128) . Yhat: the query is rotated
// once, quantized values are accumulated in the rotated domain, and the merged quantized
// accumulator is rotated back once at the end; ring tokens stay in the original domain.
#include <float.h>

#include <atomic>

#include "kvq_device.h"

namespace kvq {

namespace {

constexpr int kG = 4;                 // query heads per KV head handled by this kernel
constexpr float kNegBig = -1.0e30f;   // "no token yet" running max (finite: no inf - inf)

__device__ __forceinline__ const char* stream_cptr(const CacheGeom& g, int seq, int layer, int head, int isv)
{
    int64_t unit = ((int64_t)seq * g.n_layers + layer) * g.n_kv_heads + head;
    return g.base + unit * g.unit_bytes + (isv ? g.v_offset : 0);
}

__device__ __forceinline__ float dpp_xor1(float x) { return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)); }
__device__ __forceinline__ float dpp_xor2(float x) { return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false)); }
// row_half_mirror: lane i <-> 7-i inside each group of 8 lanes
__device__ __forceinline__ float dpp_hmirror(float x) { return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false)); }

// Sum over the 8 lanes of a token slot (lanes 8k .. 8k+7), result in every lane.
__device__ __forceinline__ float sum8(float x)
{
    x += dpp_xor1(x);
    x += dpp_xor2(x);
    x += dpp_hmirror(x);
    return x;
}

// Load the 2N bytes of 16 consecutive N-bit codes (dims 16*part ...) of one row into words.
template <int N>
__device__ __forceinline__ void load_codes16(const char* row, int part, uint32_t (&w)[(N + 1) / 2])
{
    const char* p = row + 2 * N * part;
    if constexpr (N % 2 == 0) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) w[i] = ((const uint32_t*)p)[i];
    } else {
        uint32_t h[N];
#pragma unroll
        for (int i = 0; i < N; ++i) h[i] = ((const uint16_t*)p)[i];
#pragma unroll
        for (int i = 0; i < (N + 1) / 2; ++i) w[i] = h[2 * i] | ((2 * i + 1 < N ? h[2 * i + 1] : 0u) << 16);
    }
}

// Dequantized values of dims [16*part, 16*part+16) of quantized token row t.
template <int FMT>
__device__ __forceinline__ void dequant16(const char* st, const StreamLayout& L, int64_t t, int part,
                                          const float (&crow)[16], float (&x)[16])
{
    constexpr int N = fbits(FMT);
    constexpr int KIND = fkind(FMT);
    if constexpr (KIND == KIND_BF16) {
        const uint4* p = (const uint4*)(st + L.codes + t * 256 + 32 * part);
        uint4 a = p[0], b = p[1];
        uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
            x[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        }
    } else {
        uint32_t w[(N + 1) / 2];
        load_codes16<N>(st + L.codes + t * (16 * N), part, w);
        const int b = part >> 1;
        if constexpr (kind_affine(KIND)) {
            uint32_t dm = *(const uint32_t*)(st + L.scales + t * 16 + 4 * b);
            float d = fp16_to_f32(dm & 0xFFFFu), m = fp16_to_f32(dm >> 16);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float c = m + d * (float)code_at<N>(w, j);
                if constexpr (KIND == KIND_KVARN1) c *= crow[j];
                x[j] = c;
            }
        } else {
            float d = fp16_to_f32(*(const uint16_t*)(st + L.scales + t * 8 + 2 * b));
            const float off = (float)(1 << (N - 1));
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float c = ((float)code_at<N>(w, j) - off) * d;
                if constexpr (kind_paged(KIND)) c *= crow[j];
                x[j] = c;
            }
        }
    }
}

__device__ __forceinline__ void ring16(const char* st, const StreamLayout& L, int64_t slot, int part, bool f16,
                                      float (&x)[16])
{
    const uint4* p = (const uint4*)(st + L.ring + slot * 256 + 32 * part);
    uint4 a = p[0], b = p[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        x[2 * i] = canon_to_f32(w[i] & 0xFFFFu, f16);
        x[2 * i + 1] = canon_to_f32(w[i] >> 16, f16);
    }
}

// dequant16 for a format known only at run time (one uniform branch per row).
__device__ __forceinline__ void dequant16_rt(int fmt, const char* st, const StreamLayout& L, int64_t t,
                                             int part, const float (&crow)[16], float (&x)[16])
{
    switch (fmt) {
    case 0: dequant16<0>(st, L, t, part, crow, x); break;
    case 1: dequant16<1>(st, L, t, part, crow, x); break;
    case 2: dequant16<2>(st, L, t, part, crow, x); break;
    case 3: dequant16<3>(st, L, t, part, crow, x); break;
    case 4: dequant16<4>(st, L, t, part, crow, x); break;
    case 5: dequant16<5>(st, L, t, part, crow, x); break;
    case 6: dequant16<6>(st, L, t, part, crow, x); break;
    case 7: dequant16<7>(st, L, t, part, crow, x); break;
    case 8: dequant16<8>(st, L, t, part, crow, x); break;
    case 9: dequant16<9>(st, L, t, part, crow, x); break;
    case 10: dequant16<10>(st, L, t, part, crow, x); break;
    case 11: dequant16<11>(st, L, t, part, crow, x); break;
    case 12: dequant16<12>(st, L, t, part, crow, x); break;
    case 13: dequant16<13>(st, L, t, part, crow, x); break;
    case 14: dequant16<14>(st, L, t, part, crow, x); break;
    case 15: dequant16<15>(st, L, t, part, crow, x); break;
    case 16: dequant16<16>(st, L, t, part, crow, x); break;
    case 17: dequant16<17>(st, L, t, part, crow, x); break;
    case 18: dequant16<18>(st, L, t, part, crow, x); break;
    case 19: dequant16<19>(st, L, t, part, crow, x); break;
    case 20: dequant16<20>(st, L, t, part, crow, x); break;
    case 21: dequant16<21>(st, L, t, part, crow, x); break;
    case 22: dequant16<22>(st, L, t, part, crow, x); break;
    case 23: dequant16<23>(st, L, t, part, crow, x); break;
    default: dequant16<24>(st, L, t, part, crow, x); break;
    }
}

struct Online {
    float m[kG], l[kG], acc[kG][16];
};

__device__ __forceinline__ void online_step(Online& o, const float (&qr)[kG][16], const float (&k)[16],
                                            const float (&v)[16], bool valid)
{
    float s[kG];
#pragma unroll
    for (int h = 0; h < kG; ++h) {
        float ps = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) ps = fmaf(qr[h][j], k[j], ps);
        s[h] = sum8(ps);
    }
#pragma unroll
    for (int h = 0; h < kG; ++h) {
        float mn = valid ? fmaxf(o.m[h], s[h]) : o.m[h];
        float alpha = __builtin_amdgcn_exp2f(o.m[h] - mn);
        float p = valid ? __builtin_amdgcn_exp2f(s[h] - mn) : 0.0f;
        o.m[h] = mn;
        o.l[h] = o.l[h] * alpha + p;
#pragma unroll
        for (int j = 0; j < 16; ++j) o.acc[h][j] = fmaf(p, v[j], o.acc[h][j] * alpha);
    }
}

// Combine two online states (m1,l1,a1) <- (m1,l1,a1) (+) (m2,l2,a2).
__device__ __forceinline__ void combine(float& m1, float& l1, float* a1, float m2, float l2, const float* a2, int n)
{
    float M = fmaxf(m1, m2);
    float e1 = __builtin_amdgcn_exp2f(m1 - M), e2 = __builtin_amdgcn_exp2f(m2 - M);
    l1 = l1 * e1 + l2 * e2;
    for (int j = 0; j < n; ++j) a1[j] = a1[j] * e1 + a2[j] * e2;
    m1 = M;
}

// In-place unnormalized Walsh-Hadamard transform of rows [kG][128] held in LDS.
__device__ __forceinline__ void lds_fwht(float (*buf)[kD])
{
    const int tid = threadIdx.x;
    for (int h = 1; h < kD; h <<= 1) {
        __syncthreads();
        // 256 threads, kG*64 butterflies per stage
        for (int pi = tid; pi < kG * 64; pi += blockDim.x) {
            int r = pi >> 6, k = pi & 63;
            int lo = k & (h - 1);
            int i = ((k - lo) << 1) | lo;
            float a = buf[r][i], b = buf[r][i + h];
            buf[r][i] = a + b;
            buf[r][i + h] = a - b;
        }
    }
    __syncthreads();
}

// FK: key format.  FV: value format, or -1 for "a.g.fmt_v, read at run time" (the kernel for
// caches whose K and V formats differ).
template <int FK, int FV>
__global__ __launch_bounds__(256, 2) void k_decode(DecodeArgs a)
{
    constexpr int KIND = fkind(FK);
    const int fv = FV >= 0 ? FV : a.g.fmt_v;
    const bool v_kvarn = kind_paged(fkind(fv));
    __shared__ float qs[kG][kD];
    __shared__ float wm[4][kG], wl[4][kG];
    __shared__ float wacc[4][kG][kD];

    const int tid = threadIdx.x;
    const int bid = blockIdx.x;
    // ---- which (sequence, KV head, split) ------------------------------------------------
    const DecodeWork wk = decode_work(a, bid);
    const DecodeSeq& sq = a.seqs[wk.e];
    const int head = wk.head;
    const int sp = wk.sp;
    const bool quant = sp < sq.splits_q;
    const int upw = quant ? a.units_per_wg : a.units_per_wg_t;
    const int u_lo = (quant ? sp : sp - sq.splits_q) * upw;
    const int u_cnt = quant ? sq.units_q : sq.units_t;
    const int u_hi = min(u_lo + upw, u_cnt);
    const CacheGeom& g = a.g;
    const char* kst = stream_cptr(g, sq.seq, a.layer, head, 0);
    const char* vst = stream_cptr(g, sq.seq, a.layer, head, 1);

    // ---- query of the kG heads of this KV head, scaled to the log2 domain ------------------
    for (int i = tid; i < kG * kD; i += blockDim.x) {
        int hh = i / kD, d = i % kD;
        int64_t qi = ((int64_t)sq.in_idx * g.n_q_heads + head * kG + hh) * kD + d;
        float qv = a.q_dtype ? ((const float*)a.q)[qi] : bf16_to_f32(((const uint16_t*)a.q)[qi]);
        qs[hh][d] = qv * a.scale_log2;
    }
    __syncthreads();
    if (kind_paged(KIND) && quant) {
        lds_fwht(qs);
        for (int i = tid; i < kG * kD; i += blockDim.x) qs[i / kD][i % kD] *= (1.0f / 128.0f);
        __syncthreads();
    }
    const int wave = tid >> 6, lane = tid & 63, slot = lane >> 3, part = lane & 7;
    float qr[kG][16];
#pragma unroll
    for (int h = 0; h < kG; ++h)
#pragma unroll
        for (int j = 0; j < 16; ++j) qr[h][j] = qs[h][16 * part + j];

    Online o;
#pragma unroll
    for (int h = 0; h < kG; ++h) {
        o.m[h] = kNegBig;
        o.l[h] = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) o.acc[h][j] = 0.0f;
    }

    // ---- main loop: units round-robin over the 4 waves --------------------------------------
    for (int u = u_lo + wave; u < u_hi; u += 4) {
        if (quant) {
            const int64_t t0 = (int64_t)u * kPage;
            const int64_t t1 = min<int64_t>(t0 + kPage, sq.n_q);
            float ck[16], cv[16];
            if constexpr (kind_paged(KIND)) {
                const uint16_t* cks = (const uint16_t*)(kst + g.k.cscale + (int64_t)u * 256) + 16 * part;
#pragma unroll
                for (int j = 0; j < 16; ++j) ck[j] = fp16_to_f32(cks[j]);
            }
            if (v_kvarn) {
                const uint16_t* cvs = (const uint16_t*)(vst + g.v.cscale + (int64_t)u * 256) + 16 * part;
#pragma unroll
                for (int j = 0; j < 16; ++j) cv[j] = fp16_to_f32(cvs[j]);
            }
            for (int64_t tb = t0; tb < t1; tb += 8) {
                const int64_t t = tb + slot;
                const bool valid = t < t1;
                const int64_t tc = valid ? t : t1 - 1;
                float k[16], v[16];
                dequant16<FK>(kst, g.k, tc, part, ck, k);
                if constexpr (FV >= 0) dequant16<FV>(vst, g.v, tc, part, cv, v);
                else dequant16_rt(fv, vst, g.v, tc, part, cv, v);
                online_step(o, qr, k, v, valid);
            }
        } else {
            const int64_t t0 = sq.n_q + (int64_t)u * kTailUnit;
            const int64_t t1 = min<int64_t>(t0 + kTailUnit, sq.n);
            for (int64_t tb = t0; tb < t1; tb += 8) {
                const int64_t t = tb + slot;
                const bool valid = t < t1;
                const int64_t tc = valid ? t : t1 - 1;
                const int64_t rs = tc % g.ring_slots;
                float k[16], v[16];
                ring16(kst, g.k, rs, part, g.tail_f16 != 0, k);
                ring16(vst, g.v, rs, part, g.tail_f16 != 0, v);
                online_step(o, qr, k, v, valid);
            }
        }
    }

    // ---- merge the 8 token slots of the wave (lanes with equal part) --------------------------
#pragma unroll 1
    for (int x = 8; x < 64; x <<= 1) {
#pragma unroll
        for (int h = 0; h < kG; ++h) {
            float m2 = __shfl_xor(o.m[h], x);
            float l2 = __shfl_xor(o.l[h], x);
            float a2[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) a2[j] = __shfl_xor(o.acc[h][j], x);
            combine(o.m[h], o.l[h], o.acc[h], m2, l2, a2, 16);
        }
    }
    if (slot == 0) {
#pragma unroll
        for (int h = 0; h < kG; ++h) {
#pragma unroll
            for (int j = 0; j < 16; ++j) wacc[wave][h][16 * part + j] = o.acc[h][j];
            if (part == 0) { wm[wave][h] = o.m[h]; wl[wave][h] = o.l[h]; }
        }
    }
    __syncthreads();
    // ---- merge the 4 waves, write this workgroup's partial -----------------------------------
    float* part_out = a.partials + (int64_t)wk.slot * kPartialFloats;
    for (int i = tid; i < kG * kD; i += blockDim.x) {
        const int h = i / kD, d = i % kD;
        float M = fmaxf(fmaxf(wm[0][h], wm[1][h]), fmaxf(wm[2][h], wm[3][h]));
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float ew = __builtin_amdgcn_exp2f(wm[w][h] - M);
            L += wl[w][h] * ew;
            A += wacc[w][h][d] * ew;
        }
        part_out[2 * kMaxGroup + h * kD + d] = A;
        if (d == 0) { part_out[h] = M; part_out[kMaxGroup + h] = L; }
    }
}

// Pairs with a bf16 stream (every other pair runs the fast kernel, kvq_decode_ws.hip):
// bf16 keys and values <0, 0>; bf16 keys with any value format, or quantized keys with bf16
// values, <FK, -1> (the value format is switched per block at run time).
template <int FMT>
int launch_fmt(const DecodeArgs& a, int n_wgs, hipStream_t st)
{
    if (FMT == 0 && a.g.fmt_v == 0) hipLaunchKernelGGL((k_decode<0, 0>), dim3(n_wgs), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_decode<FMT, -1>), dim3(n_wgs), dim3(256), 0, st, a);
    return (int)hipGetLastError();
}

template <int FMT>
int occ_fmt(bool mixed)
{
    int n = 0;
    hipError_t e = (FMT != 0 || mixed) ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_decode<FMT, -1>, 256, 0)
                                       : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_decode<0, 0>, 256, 0);
    return e == hipSuccess ? n : 0;
}

}  // namespace

// Caller events that bracket the split kernel (kv_debug_decode_events), or null.
static std::atomic<hipEvent_t> g_ev_before{nullptr}, g_ev_after{nullptr};

int set_decode_events(void* before, void* after)
{
    if ((before == nullptr) != (after == nullptr)) return -1;
    g_ev_before.store((hipEvent_t)before, std::memory_order_release);
    g_ev_after.store((hipEvent_t)after, std::memory_order_release);
    return 0;
}

int launch_decode(const DecodeArgs& a, int n_wgs, void* stream)
{
    const hipEvent_t eb = g_ev_before.load(std::memory_order_acquire);
    const hipEvent_t ea = g_ev_after.load(std::memory_order_acquire);
    if (eb && hipEventRecord(eb, (hipStream_t)stream) != hipSuccess) return (int)hipErrorLaunchFailure;
    int rc = launch_decode_split(a, n_wgs, stream);
    if (rc) return rc;
    if (ea && hipEventRecord(ea, (hipStream_t)stream) != hipSuccess) return (int)hipErrorLaunchFailure;
    return launch_merge(a, stream);
}

int launch_decode_split(const DecodeArgs& a, int n_wgs, void* stream)
{
    if (decode_fast_supported(a.g.fmt_k, a.g.fmt_v)) return launch_decode_fast(a, n_wgs, stream);
    hipStream_t st = (hipStream_t)stream;
    switch (a.g.fmt_k) {
    case 0: return launch_fmt<0>(a, n_wgs, st);
    case 1: return launch_fmt<1>(a, n_wgs, st);
    case 2: return launch_fmt<2>(a, n_wgs, st);
    case 3: return launch_fmt<3>(a, n_wgs, st);
    case 4: return launch_fmt<4>(a, n_wgs, st);
    case 5: return launch_fmt<5>(a, n_wgs, st);
    case 6: return launch_fmt<6>(a, n_wgs, st);
    case 7: return launch_fmt<7>(a, n_wgs, st);
    case 8: return launch_fmt<8>(a, n_wgs, st);
    case 9: return launch_fmt<9>(a, n_wgs, st);
    case 10: return launch_fmt<10>(a, n_wgs, st);
    case 11: return launch_fmt<11>(a, n_wgs, st);
    case 12: return launch_fmt<12>(a, n_wgs, st);
    case 13: return launch_fmt<13>(a, n_wgs, st);
    case 14: return launch_fmt<14>(a, n_wgs, st);
    case 15: return launch_fmt<15>(a, n_wgs, st);
    case 16: return launch_fmt<16>(a, n_wgs, st);
    case 17: return launch_fmt<17>(a, n_wgs, st);
    case 18: return launch_fmt<18>(a, n_wgs, st);
    case 19: return launch_fmt<19>(a, n_wgs, st);
    case 20: return launch_fmt<20>(a, n_wgs, st);
    case 21: return launch_fmt<21>(a, n_wgs, st);
    case 22: return launch_fmt<22>(a, n_wgs, st);
    case 23: return launch_fmt<23>(a, n_wgs, st);
    case 24: return launch_fmt<24>(a, n_wgs, st);
    default: return (int)hipErrorInvalidValue;
    }
}

int decode_wgs_per_cu(int fmt_k, int fmt_v, int group)
{
    (void)group;
    if (decode_fast_supported(fmt_k, fmt_v)) return decode_fast_wgs_per_cu(fmt_k, fmt_v);
    static int cache[kNumFormats][2] = {{0}};
    if (fmt_k < 0 || fmt_k >= kNumFormats || fmt_v < 0 || fmt_v >= kNumFormats) return 0;
    const int mx = fmt_v != fmt_k ? 1 : 0;
    if (cache[fmt_k][mx]) return cache[fmt_k][mx];
    int n = 0;
    switch (fmt_k) {
    case 0: n = occ_fmt<0>(mx); break;
    case 1: n = occ_fmt<1>(mx); break;
    case 2: n = occ_fmt<2>(mx); break;
    case 3: n = occ_fmt<3>(mx); break;
    case 4: n = occ_fmt<4>(mx); break;
    case 5: n = occ_fmt<5>(mx); break;
    case 6: n = occ_fmt<6>(mx); break;
    case 7: n = occ_fmt<7>(mx); break;
    case 8: n = occ_fmt<8>(mx); break;
    case 9: n = occ_fmt<9>(mx); break;
    case 10: n = occ_fmt<10>(mx); break;
    case 11: n = occ_fmt<11>(mx); break;
    case 12: n = occ_fmt<12>(mx); break;
    case 13: n = occ_fmt<13>(mx); break;
    case 14: n = occ_fmt<14>(mx); break;
    case 15: n = occ_fmt<15>(mx); break;
    case 16: n = occ_fmt<16>(mx); break;
    case 17: n = occ_fmt<17>(mx); break;
    case 18: n = occ_fmt<18>(mx); break;
    case 19: n = occ_fmt<19>(mx); break;
    case 20: n = occ_fmt<20>(mx); break;
    case 21: n = occ_fmt<21>(mx); break;
    case 22: n = occ_fmt<22>(mx); break;
    case 23: n = occ_fmt<23>(mx); break;
    case 24: n = occ_fmt<24>(mx); break;
    default: break;
    }
    cache[fmt_k][mx] = n;
    return n;
}

int device_cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    static int cache[64] = {0};
    if (dev < 0 || dev >= 64) return 0;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}

// ------------------------------------------------------------------------------------------
// Attention fidelity: per query head h, KL(P || Q) with P_t = softmax_t(s_t), s_t = scale
// q_h . k_t over the exact BF16 keys, and Q_t the same over the keys the cache holds
// (dequantized rows below n_q, the BF16 ring above).  With D_t = s_t - s'_t and any
// constant c,
//   KL = sum_t P_t (D_t - c) + log sum_t P_t e^{-(D_t - c)}.
// Two passes over the keys.  The first accumulates m = max s, l = sum e^{s - m} and
// A = sum e^{s - m} D, which give c = E_P[D] per head (a weighted mean: no cancellation).
// The second accumulates A = sum e^{s - m} (D - c) and B = sum e^{s - m} (e^{-(D - c)} - 1)
// with that c, so that KL = A / L + log1p(B / L) adds two small terms: quantization can
// shift every score by nearly the same amount (a common bias of the keys along q), and
// measured from any other reference both terms would be large and cancel.  A model-free
// analogue of the KL-divergence quality measure ("BeeLLama.cpp v0.4.0: KVarN, KV 정밀도
// 테일", the KLD table; "Экспериментальные методы квантизации KV-кэша в BeeLLama.cpp
// v0.4.0", the section on measuring quality): the same statistic, on attention weights
// instead of output tokens.
namespace {

struct KldState { float m, l, A, B; };

__device__ __forceinline__ void kld_add(KldState& st, float s, float e, bool valid)
{
    if (!valid) return;
    const float mn = fmaxf(st.m, s);
    const float r = expf(st.m - mn), w = expf(s - mn);
    st.l = fmaf(st.l, r, w);
    st.A = fmaf(st.A, r, w * e);
    // (a token whose cache score exceeds the exact one by more than 60 nats over c counts
    // as 60: no overflow; such a cache is far off in any case)
    st.B = fmaf(st.B, r, w * expm1f(fminf(-e, 60.0f)));
    st.m = mn;
}

__device__ __forceinline__ void kld_combine(KldState& a, const KldState& b)
{
    const float M = fmaxf(a.m, b.m);
    const float ea = expf(a.m - M), eb = expf(b.m - M);
    a.l = a.l * ea + b.l * eb;
    a.A = a.A * ea + b.A * eb;
    a.B = a.B * ea + b.B * eb;
    a.m = M;
}

template <int FK>
__global__ __launch_bounds__(256) void k_kld(KldArgs a)
{
    constexpr int KIND = fkind(FK);
    __shared__ float qs[kG][kD], qrot[kG][kD];
    __shared__ KldState ws[4][kG];
    const int tid = threadIdx.x;
    const int head = blockIdx.x / a.splits, sp = blockIdx.x % a.splits;
    const CacheGeom& g = a.g;
    const char* kst = stream_cptr(g, a.seq, a.layer, head, 0);
    for (int i = tid; i < kG * kD; i += blockDim.x) {
        const int hh = i / kD, d = i % kD;
        const int64_t qi = (int64_t)(head * kG + hh) * kD + d;
        const float qv = (a.q_dtype ? ((const float*)a.q)[qi] : bf16_to_f32(((const uint16_t*)a.q)[qi])) * a.scale;
        qs[hh][d] = qv;
        qrot[hh][d] = qv;
    }
    __syncthreads();
    if (kind_paged(KIND)) {
        lds_fwht(qrot);
        for (int i = tid; i < kG * kD; i += blockDim.x) qrot[i / kD][i % kD] *= (1.0f / 128.0f);
        __syncthreads();
    }
    const int wave = tid >> 6, lane = tid & 63, slot = lane >> 3, part = lane & 7;
    float qo[kG][16], qc[kG][16];
#pragma unroll
    for (int h = 0; h < kG; ++h)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            qo[h][j] = qs[h][16 * part + j];
            qc[h][j] = qrot[h][16 * part + j];
        }
    KldState st[kG];
#pragma unroll
    for (int h = 0; h < kG; ++h) st[h] = {kNegBig, 0.0f, 0.0f, 0.0f};
    float cref[kG];                          // pass 2: c = E_P[D] of the head (pass 1: 0)
#pragma unroll
    for (int h = 0; h < kG; ++h) cref[h] = a.pass ? a.cref[head * kG + h] : 0.0f;
    const int64_t t0 = (int64_t)sp * kKldTokens, t1 = min<int64_t>(t0 + kKldTokens, a.n);
    for (int64_t tb = t0 + 8 * wave; tb < t1; tb += 32) {
        const int64_t t = tb + slot;
        const bool valid = t < t1;
        const int64_t tc = valid ? t : t1 - 1;
        float k[16], kx[16];
        const bool quant = tc < a.n_q;
        if (quant) {
            float ck[16];
            if constexpr (kind_paged(KIND)) {
                const uint16_t* cks = (const uint16_t*)(kst + g.k.cscale + (tc / kPage) * 256) + 16 * part;
#pragma unroll
                for (int j = 0; j < 16; ++j) ck[j] = fp16_to_f32(cks[j]);
            }
            dequant16<FK>(kst, g.k, tc, part, ck, k);
        } else {
            ring16(kst, g.k, tc % g.ring_slots, part, g.tail_f16 != 0, k);
        }
        {
            const uint4* pr = (const uint4*)(a.k_ref + (tc * g.n_kv_heads + head) * kD + 16 * part);
            const uint4 w0 = pr[0], w1 = pr[1];
            const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                kx[2 * i] = canon_to_f32(ww[i] & 0xFFFFu, g.tail_f16 != 0);
                kx[2 * i + 1] = canon_to_f32(ww[i] >> 16, g.tail_f16 != 0);
            }
        }
#pragma unroll
        for (int h = 0; h < kG; ++h) {
            float se = 0.0f, sq = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                se = fmaf(qo[h][j], kx[j], se);
                sq = fmaf((kind_paged(KIND) && quant) ? qc[h][j] : qo[h][j], k[j], sq);
            }
            se = sum8(se);
            sq = sum8(sq);
            kld_add(st[h], se, (se - sq) - cref[h], valid);
        }
    }
    // slots of a wave (lanes 8 apart hold different slots; the 8 lanes of a slot agree)
#pragma unroll
    for (int h = 0; h < kG; ++h)
#pragma unroll
        for (int o = 8; o < 64; o <<= 1) {
            KldState b = {__shfl_xor(st[h].m, o), __shfl_xor(st[h].l, o), __shfl_xor(st[h].A, o),
                          __shfl_xor(st[h].B, o)};
            kld_combine(st[h], b);
        }
    if (lane == 0)
#pragma unroll
        for (int h = 0; h < kG; ++h) ws[wave][h] = st[h];
    __syncthreads();
    if (tid < kG) {
        KldState r = ws[0][tid];
        for (int w = 1; w < 4; ++w) kld_combine(r, ws[w][tid]);
        float* pp = a.partials + (((int64_t)head * a.splits + sp) * kMaxGroup + tid) * 4;
        pp[0] = r.m; pp[1] = r.l; pp[2] = r.A; pp[3] = r.B;
    }
}

// One thread per query head: merge the splits; pass 1 leaves c = A / L, pass 2 writes
// KL = A / L + log1p(B / L).
__global__ __launch_bounds__(64) void k_kld_merge(KldArgs a)
{
    const int qh = blockIdx.x * 64 + threadIdx.x;
    if (qh >= a.g.n_q_heads) return;
    const int head = qh / kG, h = qh % kG;
    KldState r = {kNegBig, 0.0f, 0.0f, 0.0f};
    for (int sp = 0; sp < a.splits; ++sp) {
        const float* pp = a.partials + (((int64_t)head * a.splits + sp) * kMaxGroup + h) * 4;
        kld_combine(r, KldState{pp[0], pp[1], pp[2], pp[3]});
    }
    if (a.pass == 0) a.cref[qh] = r.A / r.l;
    else a.out[qh] = r.A / r.l + log1pf(r.B / r.l);
}

template <int F>
int launch_kld_fmt(const KldArgs& a, hipStream_t st)
{
    hipLaunchKernelGGL(k_kld<F>, dim3(a.g.n_kv_heads * a.splits), dim3(256), 0, st, a);
    return (int)hipGetLastError();
}

int launch_kld_pass(const KldArgs& a, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    int rc;
    switch (a.g.fmt_k) {
    case 0: rc = launch_kld_fmt<0>(a, st); break;
    case 1: rc = launch_kld_fmt<1>(a, st); break;
    case 2: rc = launch_kld_fmt<2>(a, st); break;
    case 3: rc = launch_kld_fmt<3>(a, st); break;
    case 4: rc = launch_kld_fmt<4>(a, st); break;
    case 5: rc = launch_kld_fmt<5>(a, st); break;
    case 6: rc = launch_kld_fmt<6>(a, st); break;
    case 7: rc = launch_kld_fmt<7>(a, st); break;
    case 8: rc = launch_kld_fmt<8>(a, st); break;
    case 9: rc = launch_kld_fmt<9>(a, st); break;
    case 10: rc = launch_kld_fmt<10>(a, st); break;
    case 11: rc = launch_kld_fmt<11>(a, st); break;
    case 12: rc = launch_kld_fmt<12>(a, st); break;
    case 13: rc = launch_kld_fmt<13>(a, st); break;
    case 14: rc = launch_kld_fmt<14>(a, st); break;
    case 15: rc = launch_kld_fmt<15>(a, st); break;
    case 16: rc = launch_kld_fmt<16>(a, st); break;
    case 17: rc = launch_kld_fmt<17>(a, st); break;
    case 18: rc = launch_kld_fmt<18>(a, st); break;
    case 19: rc = launch_kld_fmt<19>(a, st); break;
    case 20: rc = launch_kld_fmt<20>(a, st); break;
    case 21: rc = launch_kld_fmt<21>(a, st); break;
    case 22: rc = launch_kld_fmt<22>(a, st); break;
    case 23: rc = launch_kld_fmt<23>(a, st); break;
    case 24: rc = launch_kld_fmt<24>(a, st); break;
    default: return (int)hipErrorInvalidValue;
    }
    if (rc) return rc;
    hipLaunchKernelGGL(k_kld_merge, dim3((a.g.n_q_heads + 63) / 64), dim3(64), 0, st, a);
    return (int)hipGetLastError();
}

}  // namespace

int launch_kld(const KldArgs& args, void* stream)
{
    KldArgs a = args;
    for (a.pass = 0; a.pass < 2; ++a.pass) {
        const int rc = launch_kld_pass(a, stream);
        if (rc) return rc;
    }
    return 0;
}

}  // namespace kvq
