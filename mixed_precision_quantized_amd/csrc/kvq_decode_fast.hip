// kvq_decode_fast.hip -- fast decode attention for 4-bit caches (q4_0, q4_1, kvarn4), gfx950.
//
// Same work split and merge as the generic kernel (kvq_decode.hip): 128-token quantized
// pages and 32-token ring chunks, balanced splits, a fused last-workgroup merge.  The
// quantized hot loop is rebuilt around the packed integer / fp16 dot instructions so that
// the vector ALU keeps up with HBM:
//
//  K (scores): every lane owns one 32-dim block of a token pair (4 lanes per pair, 16 pairs
//    per wave).  Codes become signed nibbles u-8 with one XOR; the query of each head is a
//    16-bit fixed-point vector per 32-dim block (scale S = max|q|/30583), split into four
//    signed 4-bit digits, so q.k over 8 dims is four v_dot8_i32_i4 with exact integer sums.
//    Lane k of a quad holds the partial sums of head (k xor r) in slot r, so a two-step DPP
//    reduce-scatter leaves lane k with the full score of head k.
//  Softmax: one running max per head shared by the whole wave; the accumulators are
//    rescaled only when a wave-wide maximum grows.  Probabilities go to LDS.
//  V (values): 8 lanes per token pair, 16 dims per lane.  Codes of the two tokens are
//    interleaved with v_perm so each 32-bit word holds (u_t0, u_t1) as two binary16
//    subnormals u*2^-24; v_dot2_f32_f16 with the binary16 weights (p*d_t0, p*d_t1) adds both
//    tokens at once.  The code offset is removed exactly from the running weight sums.
//  KVarN: keys are scored in the rotated domain with q'' = (H q / 128) * c_K of the page;
//    values accumulate in the rotated domain, scaled by the page's c_V, rotated back once
//    in the final merge (x = H Yhat / 128, H the unnormalized Sylvester Hadamard matrix).
#include <float.h>

#include "kvq_device.h"

namespace kvq {

namespace {

constexpr int kG = 4;
constexpr float kNeg = -1.0e30f;
constexpr float kQLim = 30583.0f;       // |q_int| bound so that q_int + 34952 fits 16 bits
constexpr int kQBias = 34952;           // 8 * (1 + 16 + 256 + 4096): four digits of offset 8
constexpr float kSub = 5.9604644775390625e-08f;   // 2^-24: unit of an fp16 subnormal code

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ const char* sptr(const CacheGeom& g, int seq, int layer, int head, int isv)
{
    int64_t unit = ((int64_t)seq * g.n_layers + layer) * g.n_kv_heads + head;
    return g.base + unit * g.unit_bytes + (isv ? g.v_offset : 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int QP_XOR1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int QP_XOR2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int ROW_ROR4 = 0x124;     // row_ror:4
constexpr int ROW_ROR8 = 0x128;     // row_ror:8
constexpr int ROW_HMIRROR = 0x141;  // row_half_mirror

__device__ __forceinline__ uint32_t pack_h2(float a, float b)
{
    half2_t v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fdot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

__device__ __forceinline__ float wave_max16(float x)
{
    // max over lanes with equal (lane & 3): within rows by rotation, across rows by swizzle
    x = fmaxf(x, dpp<ROW_ROR4>(x));
    x = fmaxf(x, dpp<ROW_ROR8>(x));
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

constexpr int kStages = 3;              // LDS ring depth per wave (stages of 32 tokens)

// One 32-token step of one wave, staged in LDS: K and V code rows, block-scale rows and,
// for KVarN, the page's channel-scale rows.
struct alignas(16) StageBuf {
    uint8_t kc[32 * 64];
    uint8_t vc[32 * 64];
    uint8_t ks[32 * 16];
    uint8_t vs[32 * 16];
    uint16_t ck[128];
    uint16_t cv[128];
};

// Direct global -> LDS loads: lane l writes its 16 (or 4) bytes at lds + 16 l (4 l).
// Issued from inline assembly so that the compiler does not attach a full vmcnt(0) wait to
// every later LDS read (it cannot tell which ring slot a load targets); the ring's waits are
// explicit (wait_vmcnt).  The assembly writes no VGPR (the data goes to LDS), sets M0 to the
// wave-uniform LDS address in the same block, and the address VGPRs are read at issue.
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_load16(const void* gsrc, void* lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off\n\ts_nop 0"
                 :: "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds))) : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(const void* gsrc, void* lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off\n\ts_nop 0"
                 :: "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds))) : "memory", "m0");
}

// s_waitcnt vmcnt(N) only (gfx9 encoding: vmcnt in bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

struct alignas(16) WaveLds {
    uint32_t qdig[4][4][4][4];   // [block kb][slot r][digit k][dword i]
    float qS[4][4];              // [kb][r]: fixed-point scale of head kb^r on block kb
    float qsum[4][4];            // [kb][r]: sum of the query over the block (affine format)
    float p[16][4][2];           // [pair slot][head][token]: probabilities of the iteration
};

// Fixed-point digits of the query for one page (or the whole split): 64 lanes, lane = head
// h (lane >> 4) x 8-dim group g8 (lane & 15).  src[h][d] is the scaled (and for KVarN
// rotated) query; c (nullable) the page's key channel scales.
template <bool AFFINE>
__device__ __forceinline__ void build_qdigits(WaveLds& W, const float (*src)[kD], const uint16_t* c, int lane)
{
    const int h = lane >> 4, g8 = lane & 15, kb = g8 >> 2, i = g8 & 3;
    float v[8];
    uint4 cw = c ? *(const uint4*)(c + 8 * g8) : make_uint4(0, 0, 0, 0);
    uint32_t cc[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float q = src[h][8 * g8 + e];
        if (c) q *= fp16_to_f32((cc[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        v[e] = q;
    }
    float amax = 0.0f, sum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { amax = fmaxf(amax, fabsf(v[e])); sum += v[e]; }
    amax = fmaxf(amax, dpp<QP_XOR1>(amax));
    amax = fmaxf(amax, dpp<QP_XOR2>(amax));
    if (AFFINE) {
        sum += dpp<QP_XOR1>(sum);
        sum += dpp<QP_XOR2>(sum);
    }
    const float inv = amax > 0.0f ? kQLim / amax : 0.0f;
    uint32_t d0 = 0, d1 = 0, d2 = 0, d3 = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        int qi = (int)__builtin_rintf(v[e] * inv) + kQBias;      // 0 .. 65535
        d0 |= (((uint32_t)qi & 15u) ^ 8u) << (4 * e);
        d1 |= ((((uint32_t)qi >> 4) & 15u) ^ 8u) << (4 * e);
        d2 |= ((((uint32_t)qi >> 8) & 15u) ^ 8u) << (4 * e);
        d3 |= ((((uint32_t)qi >> 12) & 15u) ^ 8u) << (4 * e);
    }
    const int r = h ^ kb;
    W.qdig[kb][r][0][i] = d0;
    W.qdig[kb][r][1][i] = d1;
    W.qdig[kb][r][2][i] = d2;
    W.qdig[kb][r][3][i] = d3;
    if (i == 0) {
        W.qS[kb][r] = amax / kQLim;
        W.qsum[kb][r] = sum;
    }
}

__device__ __forceinline__ void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// In-place unnormalized Walsh-Hadamard transform of rows [kG][128] held in LDS.
__device__ __forceinline__ void lds_fwht4(float (*buf)[kD])
{
    const int tid = threadIdx.x;
    for (int h = 1; h < kD; h <<= 1) {
        __syncthreads();
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

template <int FMT>
__global__ __launch_bounds__(256, 2) void k_decode_fast(DecodeArgs a)
{
    constexpr int KIND = fkind(FMT);
    constexpr bool KVARN = KIND == KIND_KVARN;
    constexpr bool AFF = KIND == KIND_Q1;
    constexpr int SB = AFF ? 16 : 8;            // scale bytes per token row
    static_assert(fbits(FMT) == 4, "4-bit formats only");

    __shared__ float qs[kG][kD];
    __shared__ WaveLds wl[4];
    __shared__ float wm_s[4][kG], wl_s[4][kG];
    __shared__ StageBuf stg[4][kStages];        // per-wave ring; reused by the merges
    __shared__ int last_flag;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bid = blockIdx.x;
    int e = 0;
    for (int i = 1; i < a.n_seqs; ++i)
        if (a.seqs[i].wg_base <= bid) e = i;
    const DecodeSeq& sq = a.seqs[e];
    const int S = sq.splits_q + sq.splits_t;
    const int rr = bid - sq.wg_base;
    const int head = rr / S;
    const int sp = rr % S;
    const bool quant = sp < sq.splits_q;
    const int u_lo = (quant ? sp : sp - sq.splits_q) * a.units_per_wg;
    const int u_hi = min(u_lo + a.units_per_wg, quant ? sq.units_q : sq.units_t);
    const CacheGeom& g = a.g;
    const char* kst = sptr(g, sq.seq, a.layer, head, 0);
    const char* vst = sptr(g, sq.seq, a.layer, head, 1);

    for (int i = tid; i < kG * kD; i += blockDim.x) {
        int hh = i / kD, d = i % kD;
        int64_t qi = ((int64_t)sq.in_idx * g.n_q_heads + head * kG + hh) * kD + d;
        float qv = a.q_dtype ? ((const float*)a.q)[qi] : bf16_to_f32(((const uint16_t*)a.q)[qi]);
        qs[hh][d] = qv * a.scale_log2;
    }
    __syncthreads();
    if (KVARN && quant) {
        lds_fwht4(qs);
        for (int i = tid; i < kG * kD; i += blockDim.x) qs[i / kD][i % kD] *= (1.0f / 128.0f);
        __syncthreads();
    }

    // ---- per-lane state ----------------------------------------------------------------
    const int kg = lane >> 2, kb = lane & 3;        // K layout: pair slot, block
    const int vg = lane >> 3, vp = lane & 7;        // V layout: pair slot (of 8), 16-dim part
    const int vb = vp >> 1;
    float m[kG];                                    // wave-uniform running max per head
    float lsum = 0.0f;                              // sum of p for head kb (K layout)
    float acc[kG][16];                              // V layout, raw units (x 2^-24)
    float wsum[kG];                                 // sum of fp16 weights (code offset)
    float msum[kG];                                 // affine: sum of p*(m + 8d)
#pragma unroll
    for (int h = 0; h < kG; ++h) {
        m[h] = kNeg;
        wsum[h] = 0.0f;
        msum[h] = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[h][j] = 0.0f;
    }
    float cv[16];                                   // KVarN: value channel scales of the page
#pragma unroll
    for (int j = 0; j < 16; ++j) cv[j] = 1.0f;
    WaveLds& W = wl[wave];

    if (quant) {
        uint32_t qd[4][4][4];                       // [slot r][digit][dword]
        float qS[4], qsm[4];
        auto load_digits = [&]() {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint4 w4 = *(const uint4*)&W.qdig[kb][r][k][0];
                    qd[r][k][0] = w4.x; qd[r][k][1] = w4.y; qd[r][k][2] = w4.z; qd[r][k][3] = w4.w;
                }
                qS[r] = W.qS[kb][r];
                qsm[r] = W.qsum[kb][r];
            }
        };
        if (!KVARN) {
            build_qdigits<AFF>(W, qs, nullptr, lane);
            wave_sync_lds();
            load_digits();
        }
        // Iterations of this wave: 32-token steps over its units u_lo + wave + 4i; only the
        // last quantized page of a sequence can be shorter than 128 tokens.
        const int u_first = u_lo + wave;
        const int n_units = u_first < u_hi ? (u_hi - u_first + 3) / 4 : 0;
        int J = 0;
        if (n_units > 0) {
            const int u_last = u_first + 4 * (n_units - 1);
            const int64_t last_len = min<int64_t>((int64_t)u_last * kPage + kPage, sq.n_q) - (int64_t)u_last * kPage;
            J = 4 * (n_units - 1) + (int)((last_len + 31) / 32);
        }
        const char* kcb = kst + g.k.codes;
        const char* vcb = vst + g.v.codes;
        const char* ksb = kst + g.k.scales;
        const char* vsb = vst + g.v.scales;
        // Stage j -> LDS ring slot j % kStages, always the same number of load instructions
        // (stages past the end repeat the last one), so one vmcnt value covers a stage.
        auto issue = [&](int j) {
            const int jj = j < J ? j : J - 1;
            const int u = u_first + 4 * (jj >> 2);
            const int64_t tp = (int64_t)u * kPage;
            const int64_t te = min<int64_t>(tp + kPage, sq.n_q);
            const int64_t tb = tp + 32 * (jj & 3);
            StageBuf& B = stg[wave][j % kStages];
            int64_t r = min<int64_t>(tb + (lane >> 2), te - 1);
            lds_load16(kcb + r * 64 + 16 * (lane & 3), B.kc);
            lds_load16(vcb + r * 64 + 16 * (lane & 3), B.vc);
            r = min<int64_t>(tb + 16 + (lane >> 2), te - 1);
            lds_load16(kcb + r * 64 + 16 * (lane & 3), B.kc + 1024);
            lds_load16(vcb + r * 64 + 16 * (lane & 3), B.vc + 1024);
            if (AFF) {
                r = min<int64_t>(tb + (lane & 31), te - 1);
                if (lane < 32) lds_load16(ksb + r * 16, B.ks);
                if (lane < 32) lds_load16(vsb + r * 16, B.vs);
            } else {
                r = min<int64_t>(tb + (lane >> 1), te - 1);
                lds_load4(ksb + r * 8 + 4 * (lane & 1), B.ks);
                lds_load4(vsb + r * 8 + 4 * (lane & 1), B.vs);
            }
            if (KVARN) {
                if (lane < 16) lds_load16(kst + g.k.cscale + (int64_t)u * 256 + 16 * lane, B.ck);
                if (lane < 16) lds_load16(vst + g.v.cscale + (int64_t)u * 256 + 16 * lane, B.cv);
            }
        };
        constexpr int kLoads = KVARN ? 8 : 6;
        if (J > 0) {
#pragma unroll
            for (int j = 0; j < kStages - 1; ++j) issue(j);
        }
        bool first_page = true;
#pragma unroll 1
        for (int j = 0; j < J; ++j) {
            issue(j + kStages - 1);
            wait_vmcnt<(kStages - 1) * kLoads>();     // stage j has landed in LDS
            asm volatile("" ::: "memory");
            const StageBuf& B = stg[wave][j % kStages];
            const int it = j & 3;
            const int u = u_first + 4 * (j >> 2);
            const int64_t t_page = (int64_t)u * kPage;
            const int64_t t_end = min<int64_t>(t_page + kPage, sq.n_q);
            const int64_t tb = t_page + 32 * it;
            if (KVARN && it == 0) {
                // key channel scales of the page -> query digits
                wave_sync_lds();
                build_qdigits<false>(W, qs, B.ck, lane);
                wave_sync_lds();
                load_digits();
                // value channel scales: rescale the accumulator to this page's c_V
                uint4 c0 = *(const uint4*)(B.cv + 16 * vp), c1 = *(const uint4*)(B.cv + 16 * vp + 8);
                uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
                float cn[16];
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) cn[jj] = fp16_to_f32((cw[jj >> 1] >> (16 * (jj & 1))) & 0xFFFFu);
                if (!first_page) {
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) {
                        float r = cv[jj] * __builtin_amdgcn_rcpf(cn[jj]);
#pragma unroll
                        for (int h = 0; h < kG; ++h) acc[h][jj] = fmaf(-8.0f * kSub, wsum[h], acc[h][jj]) * r;
                    }
#pragma unroll
                    for (int h = 0; h < kG; ++h) wsum[h] = 0.0f;
                }
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) cv[jj] = cn[jj];
                first_page = false;
            }
            // ---------------- K phase ----------------
            const int64_t t0 = tb + 2 * kg;
            const bool v0 = t0 < t_end, v1 = t0 + 1 < t_end;
            uint4 kc0 = *(const uint4*)(B.kc + 128 * kg + 16 * kb);
            uint4 kc1 = *(const uint4*)(B.kc + 128 * kg + 64 + 16 * kb);
            float kd0, kd1, km0 = 0.0f, km1 = 0.0f;
            if (AFF) {
                uint32_t s0 = ((const uint32_t*)B.ks)[8 * kg + kb];
                uint32_t s1 = ((const uint32_t*)B.ks)[8 * kg + 4 + kb];
                kd0 = fp16_to_f32(s0 & 0xFFFFu); kd1 = fp16_to_f32(s1 & 0xFFFFu);
                km0 = fp16_to_f32(s0 >> 16); km1 = fp16_to_f32(s1 >> 16);
            } else {
                kd0 = fp16_to_f32(((const uint16_t*)B.ks)[8 * kg + kb]);
                kd1 = fp16_to_f32(((const uint16_t*)B.ks)[8 * kg + 4 + kb]);
            }
            uint32_t c0[4] = {kc0.x ^ 0x88888888u, kc0.y ^ 0x88888888u, kc0.z ^ 0x88888888u, kc0.w ^ 0x88888888u};
            uint32_t c1[4] = {kc1.x ^ 0x88888888u, kc1.y ^ 0x88888888u, kc1.z ^ 0x88888888u, kc1.w ^ 0x88888888u};
            float ps0[4], ps1[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int a0[4], a1[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    int x = 0, y = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x = __builtin_amdgcn_sdot8((int)c0[i], (int)qd[r][k][i], x, false);
                        y = __builtin_amdgcn_sdot8((int)c1[i], (int)qd[r][k][i], y, false);
                    }
                    a0[k] = x;
                    a1[k] = y;
                }
                int t0i = a0[0] + (a0[1] << 4) + (a0[2] << 8) + (a0[3] << 12);
                int t1i = a1[0] + (a1[1] << 4) + (a1[2] << 8) + (a1[3] << 12);
                ps0[r] = (float)t0i * (qS[r] * kd0);
                ps1[r] = (float)t1i * (qS[r] * kd1);
                if (AFF) {
                    ps0[r] = fmaf(km0 + 8.0f * kd0, qsm[r], ps0[r]);
                    ps1[r] = fmaf(km1 + 8.0f * kd1, qsm[r], ps1[r]);
                }
            }
            // reduce-scatter over the quad: lane kb ends with head kb
            float k00 = ps0[0] + dpp<QP_XOR2>(ps0[2]);
            float k01 = ps0[1] + dpp<QP_XOR2>(ps0[3]);
            float k10 = ps1[0] + dpp<QP_XOR2>(ps1[2]);
            float k11 = ps1[1] + dpp<QP_XOR2>(ps1[3]);
            float s0 = k00 + dpp<QP_XOR1>(k01);
            float s1 = k10 + dpp<QP_XOR1>(k11);
            s0 = v0 ? s0 : kNeg;
            s1 = v1 ? s1 : kNeg;
            // wave-wide running max of head kb; rescale when it grows
            float wmax = wave_max16(fmaxf(s0, s1));
            float mh = m[0];
#pragma unroll
            for (int h = 1; h < kG; ++h) mh = (kb == h) ? m[h] : mh;
            if (__ballot(wmax > mh)) {
#pragma unroll
                for (int h = 0; h < kG; ++h) {
                    float nm = fmaxf(m[h], __shfl(wmax, h));
                    float al = __builtin_amdgcn_exp2f(m[h] - nm);
                    m[h] = nm;
                    wsum[h] *= al;
                    msum[h] *= al;
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) acc[h][jj] *= al;
                    if (kb == h) lsum *= al;
                }
                mh = m[0];
#pragma unroll
                for (int h = 1; h < kG; ++h) mh = (kb == h) ? m[h] : mh;
            }
            float p0 = v0 ? __builtin_amdgcn_exp2f(s0 - mh) : 0.0f;
            float p1 = v1 ? __builtin_amdgcn_exp2f(s1 - mh) : 0.0f;
            lsum += p0 + p1;
            *(float2*)&W.p[kg][kb][0] = make_float2(p0, p1);
            wave_sync_lds();
            // ---------------- V phase (two halves of 8 pairs) ----------------
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int slot = vg + 8 * half;
                uint2 a0 = *(const uint2*)(B.vc + 128 * slot + 8 * vp);
                uint2 a1 = *(const uint2*)(B.vc + 128 * slot + 64 + 8 * vp);
                uint32_t sv0, sv1;
                if (AFF) {
                    sv0 = ((const uint32_t*)B.vs)[8 * slot + vb];
                    sv1 = ((const uint32_t*)B.vs)[8 * slot + 4 + vb];
                } else {
                    sv0 = ((const uint16_t*)B.vs)[8 * slot + vb];
                    sv1 = ((const uint16_t*)B.vs)[8 * slot + 4 + vb];
                }
                float vd0 = fp16_to_f32(sv0 & 0xFFFFu), vd1 = fp16_to_f32(sv1 & 0xFFFFu);
                float4 pa = *(const float4*)&W.p[slot][0][0];
                float4 pb = *(const float4*)&W.p[slot][2][0];
                float pp[4][2] = {{pa.x, pa.y}, {pa.z, pa.w}, {pb.x, pb.y}, {pb.z, pb.w}};
                uint32_t wp[kG];
#pragma unroll
                for (int h = 0; h < kG; ++h) {
                    wp[h] = pack_h2(pp[h][0] * vd0, pp[h][1] * vd1);
                    wsum[h] = fdot2(wp[h], 0x3C003C00u, wsum[h]);
                    if (AFF) {
                        float mv0 = fp16_to_f32(sv0 >> 16), mv1 = fp16_to_f32(sv1 >> 16);
                        msum[h] = fmaf(pp[h][0], mv0 + 8.0f * vd0, fmaf(pp[h][1], mv1 + 8.0f * vd1, msum[h]));
                    }
                }
                uint32_t xw[2] = {a0.x, a0.y}, yw[2] = {a1.x, a1.y};
#pragma unroll
                for (int wdx = 0; wdx < 2; ++wdx) {
                    // (t0 dims 0-3 | t1 dims 0-3), (t0 dims 4-7 | t1 dims 4-7) of this word
                    uint32_t lo = __builtin_amdgcn_perm(yw[wdx], xw[wdx], 0x05040100u);
                    uint32_t hi = __builtin_amdgcn_perm(yw[wdx], xw[wdx], 0x07060302u);
#pragma unroll
                    for (int n = 0; n < 4; ++n) {
                        uint32_t pl = (lo >> (4 * n)) & 0x000F000Fu;
                        uint32_t ph = (hi >> (4 * n)) & 0x000F000Fu;
#pragma unroll
                        for (int h = 0; h < kG; ++h) {
                            acc[h][8 * wdx + n] = fdot2(wp[h], pl, acc[h][8 * wdx + n]);
                            acc[h][8 * wdx + 4 + n] = fdot2(wp[h], ph, acc[h][8 * wdx + 4 + n]);
                        }
                    }
                }
            }
            wave_sync_lds();
        }
        wait_vmcnt<0>();                             // repeated tail stages
        asm volatile("" ::: "memory");
        // raw units -> values: remove the code offset, apply 2^24 and the page's c_V
#pragma unroll
        for (int h = 0; h < kG; ++h)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                float v = fmaf(-8.0f * kSub, wsum[h], acc[h][jj]) * 16777216.0f;
                if (KVARN) v *= cv[jj];
                if (AFF) v += msum[h];
                acc[h][jj] = v;
            }
    } else {
        // ---------------- BF16 ring chunks (original domain, fp32 math) ----------------
        float qr[kG][16];
#pragma unroll
        for (int h = 0; h < kG; ++h)
#pragma unroll
            for (int j = 0; j < 16; ++j) qr[h][j] = qs[h][16 * vp + j];
        for (int u = u_lo + wave; u < u_hi; u += 4) {
            const int64_t t_lo = sq.n_q + (int64_t)u * kTailUnit;
            const int64_t t_end = min<int64_t>(t_lo + kTailUnit, sq.n);
#pragma unroll 1
            for (int64_t tb = t_lo; tb < t_end; tb += 16) {
                const int64_t t0 = tb + 2 * vg;
                const bool v0 = t0 < t_end, v1 = t0 + 1 < t_end;
                const int64_t s0r = (v0 ? t0 : t_end - 1) % g.ring_slots;
                const int64_t s1r = (v1 ? t0 + 1 : t_end - 1) % g.ring_slots;
                float k0[16], k1[16], x0[16], x1[16];
                const uint4* pk0 = (const uint4*)(kst + g.k.ring + s0r * 256 + 32 * vp);
                const uint4* pk1 = (const uint4*)(kst + g.k.ring + s1r * 256 + 32 * vp);
                const uint4* pv0 = (const uint4*)(vst + g.v.ring + s0r * 256 + 32 * vp);
                const uint4* pv1 = (const uint4*)(vst + g.v.ring + s1r * 256 + 32 * vp);
                uint4 w[8] = {pk0[0], pk0[1], pk1[0], pk1[1], pv0[0], pv0[1], pv1[0], pv1[1]};
                float* dst[4] = {k0, k1, x0, x1};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint32_t ww[8] = {w[2 * r].x, w[2 * r].y, w[2 * r].z, w[2 * r].w,
                                      w[2 * r + 1].x, w[2 * r + 1].y, w[2 * r + 1].z, w[2 * r + 1].w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        dst[r][2 * i] = bf16_to_f32(ww[i] & 0xFFFFu);
                        dst[r][2 * i + 1] = bf16_to_f32(ww[i] >> 16);
                    }
                }
                float s0[kG], s1[kG];
#pragma unroll
                for (int h = 0; h < kG; ++h) {
                    float x = 0.0f, y = 0.0f;
#pragma unroll
                    for (int j = 0; j < 16; ++j) { x = fmaf(qr[h][j], k0[j], x); y = fmaf(qr[h][j], k1[j], y); }
                    x += dpp<QP_XOR1>(x); x += dpp<QP_XOR2>(x); x += dpp<ROW_HMIRROR>(x);
                    y += dpp<QP_XOR1>(y); y += dpp<QP_XOR2>(y); y += dpp<ROW_HMIRROR>(y);
                    s0[h] = v0 ? x : kNeg;
                    s1[h] = v1 ? y : kNeg;
                }
#pragma unroll
                for (int h = 0; h < kG; ++h) {
                    float wmax = fmaxf(s0[h], s1[h]);
                    wmax = fmaxf(wmax, dpp<ROW_ROR8>(wmax));
                    wmax = fmaxf(wmax, __shfl_xor(wmax, 16));
                    wmax = fmaxf(wmax, __shfl_xor(wmax, 32));
                    if (wmax > m[h]) {           // uniform across the wave
                        float al = __builtin_amdgcn_exp2f(m[h] - wmax);
                        m[h] = wmax;
#pragma unroll
                        for (int j = 0; j < 16; ++j) acc[h][j] *= al;
                        msum[h] *= al;           // holds sum of p for head h (lanes with vp == 0)
                    }
                    float p0 = v0 ? __builtin_amdgcn_exp2f(s0[h] - m[h]) : 0.0f;
                    float p1 = v1 ? __builtin_amdgcn_exp2f(s1[h] - m[h]) : 0.0f;
                    if (vp == 0) msum[h] += p0 + p1;
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc[h][j] = fmaf(p0, x0[j], fmaf(p1, x1[j], acc[h][j]));
                }
            }
        }
    }

    // ---- wave merge: token slots share the wave max, so plain sums suffice -------------
    float lh[kG];
#pragma unroll
    for (int h = 0; h < kG; ++h) lh[h] = quant ? ((kb == h) ? lsum : 0.0f) : msum[h];
#pragma unroll
    for (int h = 0; h < kG; ++h) {
        float x = lh[h];
        x += __shfl_xor(x, 1); x += __shfl_xor(x, 2); x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8); x += __shfl_xor(x, 16); x += __shfl_xor(x, 32);
        lh[h] = x;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float y = acc[h][j];
            y += dpp<ROW_ROR8>(y);
            y += __shfl_xor(y, 16);
            y += __shfl_xor(y, 32);
            acc[h][j] = y;
        }
    }
    float (*wacc_me)[kD] = reinterpret_cast<float (*)[kD]>(&stg[wave][0]);
    if (vg == 0) {
#pragma unroll
        for (int h = 0; h < kG; ++h) {
#pragma unroll
            for (int j = 0; j < 16; ++j) wacc_me[h][16 * vp + j] = acc[h][j];
            if (vp == 0) { wm_s[wave][h] = m[h]; wl_s[wave][h] = lh[h]; }
        }
    }
    __syncthreads();
    float* part_out = a.partials + (int64_t)bid * kPartialFloats;
    for (int i = tid; i < kG * kD; i += blockDim.x) {
        const int h = i / kD, d = i % kD;
        float M = fmaxf(fmaxf(wm_s[0][h], wm_s[1][h]), fmaxf(wm_s[2][h], wm_s[3][h]));
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float ew = __builtin_amdgcn_exp2f(wm_s[w][h] - M);
            L += wl_s[w][h] * ew;
            A += reinterpret_cast<const float (*)[kD]>(&stg[w][0])[h][d] * ew;
        }
        part_out[2 * kMaxGroup + h * kD + d] = A;
        if (d == 0) { part_out[h] = M; part_out[kMaxGroup + h] = L; }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        uint32_t* ctr = a.counters + sq.in_idx * g.n_kv_heads + head;
        uint32_t old = atomicAdd(ctr, 1u);
        int last = (old == (uint32_t)(S - 1));
        if (last) *ctr = 0u;
        last_flag = last;
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();

    const int first = sq.wg_base + head * S;
    __syncthreads();                            // every wave's partial has been read
    float (*oq)[kD] = reinterpret_cast<float (*)[kD]>(&stg[0][0]);
    float (*ot)[kD] = reinterpret_cast<float (*)[kD]>(&stg[1][0]);
    for (int i = tid; i < kG * kD; i += blockDim.x) {
        const int h = i / kD, d = i % kD;
        float M = kNeg;
        for (int s = 0; s < S; ++s)
            M = fmaxf(M, __hip_atomic_load(a.partials + (int64_t)(first + s) * kPartialFloats + h,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        float L = 0.0f, Aq = 0.0f, At = 0.0f;
        for (int s = 0; s < S; ++s) {
            const float* pp = a.partials + (int64_t)(first + s) * kPartialFloats;
            float mm = __hip_atomic_load(pp + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            float ll = __hip_atomic_load(pp + kMaxGroup + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            float ac = __hip_atomic_load(pp + 2 * kMaxGroup + h * kD + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            float ew = __builtin_amdgcn_exp2f(mm - M);
            L += ll * ew;
            if (s < sq.splits_q) Aq += ac * ew; else At += ac * ew;
        }
        oq[h][d] = Aq;
        ot[h][d] = At;
        if (d == 0) wl_s[0][h] = L;
    }
    __syncthreads();
    if (KVARN) lds_fwht4(oq);
    for (int i = tid; i < kG * kD; i += blockDim.x) {
        const int h = i / kD, d = i % kD;
        float vq = oq[h][d];
        if (KVARN) vq *= (1.0f / 128.0f);
        a.out[((int64_t)sq.in_idx * g.n_q_heads + head * kG + h) * kD + d] = (vq + ot[h][d]) / wl_s[0][h];
    }
}

template <int FMT>
int launch_fast_fmt(const DecodeArgs& a, int n_wgs, hipStream_t st)
{
    hipLaunchKernelGGL(k_decode_fast<FMT>, dim3(n_wgs), dim3(256), 0, st, a);
    return (int)hipGetLastError();
}

template <int FMT>
int occ_fast()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_decode_fast<FMT>, 256, 0) != hipSuccess) return 0;
    return n;
}

}  // namespace

bool decode_fast_supported(int fmt_k, int fmt_v)
{
    return fmt_k == fmt_v && (fmt_k == 5 || fmt_k == 6 || fmt_k == 15);
}

int launch_decode_fast(const DecodeArgs& a, int n_wgs, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    switch (a.g.fmt_k) {
    case 5: return launch_fast_fmt<5>(a, n_wgs, st);
    case 6: return launch_fast_fmt<6>(a, n_wgs, st);
    case 15: return launch_fast_fmt<15>(a, n_wgs, st);
    default: return (int)hipErrorInvalidValue;
    }
}

int decode_fast_wgs_per_cu(int fmt)
{
    static int cache[19] = {0};
    if (fmt < 0 || fmt >= 19) return 0;
    if (!cache[fmt]) {
        switch (fmt) {
        case 5: cache[fmt] = occ_fast<5>(); break;
        case 6: cache[fmt] = occ_fast<6>(); break;
        case 15: cache[fmt] = occ_fast<15>(); break;
        default: return 0;
        }
    }
    return cache[fmt];
}

}  // namespace kvq
