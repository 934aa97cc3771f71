// kvq_decode_ws.hip -- fast decode attention for 4-bit caches (q4_0, q4_1, kvarn4), gfx950.
//
// Same work split as the generic kernel (kvq_decode.hip): 128-token quantized pages and
// 32-token ring chunks, balanced splits, partial results merged by kvq_merge.hip.  Inside a
// workgroup the waves specialize, so each role fits in half the registers and four waves
// share every SIMD:
//
//   waves 0,1  "K waves"  score 32 tokens per step and run the softmax;
//   waves 2,3  "V waves"  accumulate the values of the step the K waves finished before.
//
// Wave w and wave w+2 form a pair that walks every other unit of the workgroup; the pair
// hands the probabilities of a step over through a double-buffered block of LDS, and the
// whole workgroup takes one barrier per step.  Every wave streams its own rows (K codes or
// V codes, block scales and, for KVarN, the page's channel scales) through a three-deep
// LDS ring filled by direct global-to-LDS loads two steps ahead.
//
//  K: one lane per 32-dim block of a token pair.  Codes become signed nibbles u-8 with one
//     XOR; the query of each head is a 16-bit fixed-point vector per block (scale
//     S = max|q|/30583) split into four signed 4-bit digits, so q.k over 8 dims is four
//     v_dot8_i32_i4 with exact integer sums.  Lane k of a quad holds the partial sums of
//     head (k xor r) in slot r; a two-step DPP reduce-scatter leaves lane k with head k.
//     One running max per head is shared by the wave; a step whose maximum grows passes the
//     rescale factors to the V wave.
//  V: 8 lanes per token pair, 16 dims per lane.  v_perm interleaves the codes of the two
//     tokens so each word holds (u_t0, u_t1) as two binary16 subnormals u*2^-24, and
//     v_dot2_f32_f16 with the binary16 weights (p*d_t0, p*d_t1) adds both tokens at once.
//     The code offset is removed exactly with the running sum of the weights.
//  KVarN: keys are scored in the rotated domain with q'' = (H q / 128) * c_K of the page;
//     values accumulate in the rotated domain scaled by the page's c_V and are rotated back
//     once in the final merge (x = H Yhat / 128, H the unnormalized Sylvester Hadamard).
//  Ring (BF16 tail) workgroups use the same pairing with binary32 arithmetic.
#include <float.h>

#include "kvq_device.h"

namespace kvq {

namespace {

constexpr int kG = 4;
constexpr float kNeg = -1.0e30f;
constexpr float kQLim = 30583.0f;        // |q_int| bound so that q_int + 34952 fits 16 bits
constexpr int kQBias = 34952;            // 8 * (1 + 16 + 256 + 4096): offset 8 in each digit
constexpr float kSub = 5.9604644775390625e-08f;   // 2^-24: unit of a binary16 subnormal code
constexpr int kStages = 3;               // LDS ring depth per wave

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// reduction over lanes with equal (lane & 3)
__device__ __forceinline__ float wave_max16(float x)
{
    x = fmaxf(x, dpp<ROW_ROR4>(x));
    x = fmaxf(x, dpp<ROW_ROR8>(x));
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum16(float x)
{
    x += dpp<ROW_ROR4>(x);
    x += dpp<ROW_ROR8>(x);
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}
// reduction over lanes with equal (lane & 7)
__device__ __forceinline__ float wave_max8(float x)
{
    x = fmaxf(x, dpp<ROW_ROR8>(x));
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum8(float x)
{
    x += dpp<ROW_ROR8>(x);
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// Direct global -> LDS loads: lane l writes its 16 (or 4) bytes at lds + 16 l (4 l).
// Issued from inline assembly so that the compiler does not attach a full vmcnt(0) wait to
// every later LDS read (it cannot tell which ring slot a load targets); the ring's waits are
// explicit (wait_vmcnt).  The assembly writes no VGPR (the data goes to LDS), sets M0 to the
// wave-uniform LDS address in the same block, and the address VGPRs are read at issue.
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_load16(const void* gsrc, const void* lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off\n\ts_nop 0"
                 :: "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds))) : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(const void* gsrc, const void* lds)
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

__device__ __forceinline__ void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One 32-token step of one stream in LDS.  Code rows are stored even tokens first
// (rows 0..15 = tokens 0,2,..,30) then odd tokens (rows 16..31), so both the score lanes
// (16 bytes of one token) and the value lanes (8 bytes of one token) read without bank
// conflicts; block-scale rows are in token order.
struct alignas(16) Stage {
    uint8_t codes[32 * 64];
    uint8_t scales[32 * 16];
    uint16_t chan[128];
};

struct alignas(16) PBuf {
    float p[16][4][2];       // [pair slot][head][token] probabilities of the step
    float alpha[4];          // accumulator rescale of the step (running max grew)
    float pad[4];
};

struct alignas(16) QDig {
    uint32_t d[4][4][4][4];  // [block kb][slot r][digit k][dword i] of head kb^r
    float S[4][4];           // [kb][r] fixed-point scale
    float qsum[4][4];        // [kb][r] block sum of the query (affine format)
};

struct alignas(16) WsLds {
    float qs[kG][kD];
    Stage st[4][kStages];
    PBuf pb[2][2];
    QDig qd[2];
    float wm[2][kG], wl[2][kG];
};

// Fixed-point digits of the query (one page or the whole split).  Lane = head h
// (lane >> 4) x 8-dim group g8 (lane & 15).  c: the page's key channel scales or null.
template <bool AFFINE>
__device__ __forceinline__ void build_qdigits(QDig& Q, const float (*src)[kD], const uint16_t* c, int lane)
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
    const float inv = amax > 0.0f ? kQLim * __builtin_amdgcn_rcpf(amax) : 0.0f;
    uint32_t d0 = 0, d1 = 0, d2 = 0, d3 = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        int qi = (int)__builtin_rintf(fminf(fmaxf(v[e] * inv, -kQLim), kQLim)) + kQBias;
        d0 |= (((uint32_t)qi & 15u) ^ 8u) << (4 * e);
        d1 |= ((((uint32_t)qi >> 4) & 15u) ^ 8u) << (4 * e);
        d2 |= ((((uint32_t)qi >> 8) & 15u) ^ 8u) << (4 * e);
        d3 |= ((((uint32_t)qi >> 12) & 15u) ^ 8u) << (4 * e);
    }
    const int r = h ^ kb;
    Q.d[kb][r][0][i] = d0;
    Q.d[kb][r][1][i] = d1;
    Q.d[kb][r][2][i] = d2;
    Q.d[kb][r][3][i] = d3;
    if (i == 0) {
        // dequantization scale of the digits: q ~ q_int * S
        Q.S[kb][r] = inv > 0.0f ? 1.0f / inv : 0.0f;
        Q.qsum[kb][r] = sum;
    }
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
__global__ __launch_bounds__(256, 4) void k_decode_ws(DecodeArgs a)
{
    constexpr int KIND = fkind(FMT);
    constexpr bool KVARN = KIND == KIND_KVARN;
    constexpr bool AFF = KIND == KIND_Q1;
    constexpr int SB = AFF ? 16 : 8;                  // scale bytes per token row
    constexpr int kLoads = 3 + (KVARN ? 1 : 0);      // load instructions per stage
    static_assert(fbits(FMT) == 4, "4-bit formats only");
    static_assert(sizeof(Stage) * kStages >= 2 * 2 * kG * kD * sizeof(float), "merge scratch fits one wave ring");

    __shared__ WsLds S;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pr = wave & 1;                          // pair
    const bool kwave = wave < 2;
    const int bid = blockIdx.x;
    int e = 0;
    for (int i = 1; i < a.n_seqs; ++i)
        if (a.seqs[i].wg_base <= bid) e = i;
    const DecodeSeq& sq = a.seqs[e];
    const int SPL = sq.splits_q + sq.splits_t;
    const int rr = bid - sq.wg_base;
    const int head = rr / SPL;
    const int sp = rr % SPL;
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
        S.qs[hh][d] = qv * a.scale_log2;
    }
    __syncthreads();
    if (KVARN && quant) {
        lds_fwht4(S.qs);
        for (int i = tid; i < kG * kD; i += blockDim.x) S.qs[i / kD][i % kD] *= (1.0f / 128.0f);
        __syncthreads();
    }

    // steps of each pair: the pair walks units u_lo + pr + 2i
    auto steps_of = [&](int p) -> int {
        const int uf = u_lo + p;
        if (uf >= u_hi) return 0;
        const int nu = (u_hi - uf + 1) / 2;
        if (!quant) return nu;
        const int ul = uf + 2 * (nu - 1);
        const int64_t len = min<int64_t>((int64_t)ul * kPage + kPage, sq.n_q) - (int64_t)ul * kPage;
        return 4 * (nu - 1) + (int)((len + 31) / 32);
    };
    const int J = steps_of(pr);
    const int Jmax = max(steps_of(0), steps_of(1));
    const int u_first = u_lo + pr;

    const int kg = lane >> 2, kb = lane & 3;          // K layout: pair slot, block
    const int vg = lane >> 3, vp = lane & 7;          // V layout: pair slot (of 8), 16-dim part
    const int vb = vp >> 1;

    // end of a role: the K wave leaves (m, l) per head, the V wave its slot-summed accumulator
    auto finish_k = [&](float mv, float lsum, bool quant_layout) {
        const float t = quant_layout ? wave_sum16(lsum) : wave_sum8(vp < kG ? lsum : 0.0f);
        if (lane < kG) {                 // lane h holds head h in both layouts
            S.wl[pr][lane] = t;
            S.wm[pr][lane] = mv;
        }
    };
    auto finish_v = [&](float (&acc)[kG][16]) {
        float (*wacc)[kD] = reinterpret_cast<float (*)[kD]>(&S.st[wave][0]);
#pragma unroll
        for (int h = 0; h < kG; ++h)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const float y = wave_sum8(acc[h][jj]);
                if (vg == 0) wacc[h][16 * vp + jj] = y;
            }
    };
    if (quant) {
        const char* cbase = kwave ? kst + g.k.codes : vst + g.v.codes;
        const char* sbase = kwave ? kst + g.k.scales : vst + g.v.scales;
        const char* chbase = kwave ? kst + g.k.cscale : vst + g.v.cscale;
        Stage* ring = S.st[wave];
        // stage j -> ring slot j % kStages; the number of load instructions per stage is
        // fixed (stages past the end repeat the last), so one vmcnt value covers a stage.
        auto issue = [&](int j) {
            const int jj = j < J ? j : J - 1;
            const int u = u_first + 2 * (jj >> 2);
            const int64_t tp = (int64_t)u * kPage;
            const int64_t te = min<int64_t>(tp + kPage, sq.n_q);
            const int64_t tb = tp + 32 * (jj & 3);
            Stage& B = ring[j % kStages];
            int64_t r = min<int64_t>(tb + 2 * (lane >> 2), te - 1);
            lds_load16(cbase + r * 64 + 16 * (lane & 3), B.codes);
            r = min<int64_t>(tb + 2 * (lane >> 2) + 1, te - 1);
            lds_load16(cbase + r * 64 + 16 * (lane & 3), B.codes + 1024);
            if (AFF) {
                r = min<int64_t>(tb + (lane & 31), te - 1);
                if (lane < 32) lds_load16(sbase + r * 16, B.scales);
            } else {
                r = min<int64_t>(tb + (lane >> 1), te - 1);
                lds_load4(sbase + r * 8 + 4 * (lane & 1), B.scales);
            }
            if (KVARN) {
                if (lane < 16) lds_load16(chbase + (int64_t)u * 256 + 16 * lane, B.chan);
            }
        };
        if (J > 0) {
            issue(0);
            issue(1);
        }
        if (kwave) {
            // ================================ K wave ================================
            float mh = kNeg;                           // running max of the lane's head kb
            float lsum = 0.0f;                         // sum of p of the lane's head
            QDig& Q = S.qd[pr];
            uint32_t qd[4][4][4];
            float qS[4], qsm[4];
            auto load_digits = [&]() {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        uint4 w4 = *(const uint4*)&Q.d[kb][r][k][0];
                        qd[r][k][0] = w4.x; qd[r][k][1] = w4.y; qd[r][k][2] = w4.z; qd[r][k][3] = w4.w;
                    }
                    qS[r] = Q.S[kb][r];
                    qsm[r] = Q.qsum[kb][r];
                }
            };
            if (!KVARN) {
                build_qdigits<AFF>(Q, S.qs, nullptr, lane);
                wave_sync_lds();
                load_digits();
            }
            // one 32-token step of the scores; `page_start`: the step opens a page
            auto kstep = [&](int j, int64_t t_page, int64_t t_end, bool page_start) __attribute__((always_inline)) {
                issue(j + 2);
                wait_vmcnt<2 * kLoads>();
                asm volatile("" ::: "memory");
                const Stage& B = ring[j % kStages];
                if (KVARN && page_start) {
                    wave_sync_lds();
                    build_qdigits<false>(Q, S.qs, B.chan, lane);
                    wave_sync_lds();
                    load_digits();
                }
                const int64_t t0 = t_page + 32 * (j & 3) + 2 * kg;
                const bool v0 = t0 < t_end, v1 = t0 + 1 < t_end;
                const uint4 kc0 = *(const uint4*)(B.codes + 16 * lane);
                const uint4 kc1 = *(const uint4*)(B.codes + 1024 + 16 * lane);
                float kd0, kd1, km0 = 0.0f, km1 = 0.0f;
                if (AFF) {
                    uint32_t s0 = ((const uint32_t*)B.scales)[8 * kg + kb];
                    uint32_t s1 = ((const uint32_t*)B.scales)[8 * kg + 4 + kb];
                    kd0 = fp16_to_f32(s0 & 0xFFFFu); kd1 = fp16_to_f32(s1 & 0xFFFFu);
                    km0 = fp16_to_f32(s0 >> 16); km1 = fp16_to_f32(s1 >> 16);
                } else {
                    kd0 = fp16_to_f32(((const uint16_t*)B.scales)[8 * kg + kb]);
                    kd1 = fp16_to_f32(((const uint16_t*)B.scales)[8 * kg + 4 + kb]);
                }
                const uint32_t c0[4] = {kc0.x ^ 0x88888888u, kc0.y ^ 0x88888888u, kc0.z ^ 0x88888888u, kc0.w ^ 0x88888888u};
                const uint32_t c1[4] = {kc1.x ^ 0x88888888u, kc1.y ^ 0x88888888u, kc1.z ^ 0x88888888u, kc1.w ^ 0x88888888u};
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
                    const int t0i = a0[0] + (a0[1] << 4) + (a0[2] << 8) + (a0[3] << 12);
                    const int t1i = a1[0] + (a1[1] << 4) + (a1[2] << 8) + (a1[3] << 12);
                    ps0[r] = (float)t0i * (qS[r] * kd0);
                    ps1[r] = (float)t1i * (qS[r] * kd1);
                    if (AFF) {
                        ps0[r] = fmaf(km0 + 8.0f * kd0, qsm[r], ps0[r]);
                        ps1[r] = fmaf(km1 + 8.0f * kd1, qsm[r], ps1[r]);
                    }
                }
                // reduce-scatter over the quad: lane kb ends with head kb
                const float k00 = ps0[0] + dpp<QP_XOR2>(ps0[2]);
                const float k01 = ps0[1] + dpp<QP_XOR2>(ps0[3]);
                const float k10 = ps1[0] + dpp<QP_XOR2>(ps1[2]);
                const float k11 = ps1[1] + dpp<QP_XOR2>(ps1[3]);
                float s0 = k00 + dpp<QP_XOR1>(k01);
                float s1 = k10 + dpp<QP_XOR1>(k11);
                s0 = v0 ? s0 : kNeg;
                s1 = v1 ? s1 : kNeg;
                // lanes with equal kb hold the same head: the new max needs no exchange
                const float nm = fmaxf(mh, wave_max16(fmaxf(s0, s1)));
                const float al = __builtin_amdgcn_exp2f(mh - nm);    // exactly 1 if unchanged
                mh = nm;
                lsum *= al;
                const float p0 = v0 ? __builtin_amdgcn_exp2f(s0 - mh) : 0.0f;
                const float p1 = v1 ? __builtin_amdgcn_exp2f(s1 - mh) : 0.0f;
                lsum += p0 + p1;
                PBuf& P = S.pb[pr][j & 1];
                *(float2*)&P.p[kg][kb][0] = make_float2(p0, p1);
                if (lane < kG) P.alpha[lane] = al;
                __syncthreads();
            };
            // J work steps, page by page, then idle barriers up to the workgroup's Jmax + 1
            int j = 0;
#pragma unroll 1
            for (int u = u_first; u < u_hi; u += 2) {
                const int64_t t_page = (int64_t)u * kPage;
                const int64_t t_end = min<int64_t>(t_page + kPage, sq.n_q);
                const int ns = (int)((t_end - t_page + 31) / 32);
                kstep(j, t_page, t_end, true);
                ++j;
#pragma unroll 1
                for (int js = 1; js < ns; ++js, ++j) kstep(j, t_page, t_end, false);
            }
#pragma unroll 1
            for (; j <= Jmax; ++j) __syncthreads();
            finish_k(mh, lsum, true);
        } else {
            // ================================ V wave ================================
            float acc[kG][16], wsum[kG], msum[kG], cv[16];
#pragma unroll
            for (int h = 0; h < kG; ++h) {
                wsum[h] = 0.0f;
                msum[h] = 0.0f;
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) acc[h][jj] = 0.0f;
            }
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) cv[jj] = 1.0f;
            auto vstep = [&](int j, bool page_start) __attribute__((always_inline)) {
                issue(j + 2);
                wait_vmcnt<2 * kLoads>();
                asm volatile("" ::: "memory");
                const Stage& B = ring[j % kStages];
                const PBuf& P = S.pb[pr][j & 1];
                const float4 al = *(const float4*)P.alpha;
                if (al.x != 1.0f || al.y != 1.0f || al.z != 1.0f || al.w != 1.0f) {
                    const float alv[kG] = {al.x, al.y, al.z, al.w};
#pragma unroll
                    for (int h = 0; h < kG; ++h) {
                        wsum[h] *= alv[h];
                        msum[h] *= alv[h];
#pragma unroll
                        for (int jj = 0; jj < 16; ++jj) acc[h][jj] *= alv[h];
                    }
                }
                if (KVARN && page_start) {
                    // this page's value channel scales: rescale the accumulator to them (the
                    // accumulator is zero before the first page, so the first rescale is inert)
                    const uint4 c0 = *(const uint4*)(B.chan + 16 * vp);
                    const uint4 c1 = *(const uint4*)(B.chan + 16 * vp + 8);
                    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) {
                        const float cn = fp16_to_f32((cw[jj >> 1] >> (16 * (jj & 1))) & 0xFFFFu);
                        const float r = cv[jj] * __builtin_amdgcn_rcpf(cn);
#pragma unroll
                        for (int h = 0; h < kG; ++h) acc[h][jj] = fmaf(-8.0f * kSub, wsum[h], acc[h][jj]) * r;
                        cv[jj] = cn;
                    }
#pragma unroll
                    for (int h = 0; h < kG; ++h) wsum[h] = 0.0f;
                }
#pragma unroll 1
                for (int half = 0; half < 2; ++half) {
                    const int slot = vg + 8 * half;
                    const uint2 a0 = *(const uint2*)(B.codes + 64 * slot + 8 * vp);
                    const uint2 a1 = *(const uint2*)(B.codes + 1024 + 64 * slot + 8 * vp);
                    uint32_t sv0, sv1;
                    if (AFF) {
                        sv0 = ((const uint32_t*)B.scales)[8 * slot + vb];
                        sv1 = ((const uint32_t*)B.scales)[8 * slot + 4 + vb];
                    } else {
                        sv0 = ((const uint16_t*)B.scales)[8 * slot + vb];
                        sv1 = ((const uint16_t*)B.scales)[8 * slot + 4 + vb];
                    }
                    const float vd0 = fp16_to_f32(sv0 & 0xFFFFu), vd1 = fp16_to_f32(sv1 & 0xFFFFu);
                    const float4 pa = *(const float4*)&P.p[slot][0][0];
                    const float4 pb = *(const float4*)&P.p[slot][2][0];
                    const float pp[4][2] = {{pa.x, pa.y}, {pa.z, pa.w}, {pb.x, pb.y}, {pb.z, pb.w}};
                    uint32_t wp[kG];
#pragma unroll
                    for (int h = 0; h < kG; ++h) {
                        wp[h] = pack_h2(pp[h][0] * vd0, pp[h][1] * vd1);
                        wsum[h] = fdot2(wp[h], 0x3C003C00u, wsum[h]);
                        if (AFF) {
                            const float mv0 = fp16_to_f32(sv0 >> 16), mv1 = fp16_to_f32(sv1 >> 16);
                            msum[h] = fmaf(pp[h][0], mv0 + 8.0f * vd0, fmaf(pp[h][1], mv1 + 8.0f * vd1, msum[h]));
                        }
                    }
                    const uint32_t xw[2] = {a0.x, a0.y}, yw[2] = {a1.x, a1.y};
#pragma unroll
                    for (int wdx = 0; wdx < 2; ++wdx) {
                        // (t0 dims 0-3 | t1 dims 0-3) and (t0 dims 4-7 | t1 dims 4-7)
                        const uint32_t lo = __builtin_amdgcn_perm(yw[wdx], xw[wdx], 0x05040100u);
                        const uint32_t hi = __builtin_amdgcn_perm(yw[wdx], xw[wdx], 0x07060302u);
#pragma unroll
                        for (int n = 0; n < 4; ++n) {
                            const uint32_t pl = (lo >> (4 * n)) & 0x000F000Fu;
                            const uint32_t ph = (hi >> (4 * n)) & 0x000F000Fu;
#pragma unroll
                            for (int h = 0; h < kG; ++h) {
                                acc[h][8 * wdx + n] = fdot2(wp[h], pl, acc[h][8 * wdx + n]);
                                acc[h][8 * wdx + 4 + n] = fdot2(wp[h], ph, acc[h][8 * wdx + 4 + n]);
                            }
                        }
                    }
                }
                __syncthreads();
            };
            // one idle barrier (the K wave scores the first step), J work steps, idle barriers
            __syncthreads();
            int j = 0;
#pragma unroll 1
            for (int u = u_first; u < u_hi; u += 2) {
                const int64_t t_page = (int64_t)u * kPage;
                const int64_t t_end = min<int64_t>(t_page + kPage, sq.n_q);
                const int ns = (int)((t_end - t_page + 31) / 32);
                vstep(j, true);
                ++j;
#pragma unroll 1
                for (int js = 1; js < ns; ++js, ++j) vstep(j, false);
            }
#pragma unroll 1
            for (++j; j <= Jmax; ++j) __syncthreads();
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
            wait_vmcnt<0>();                          // stages past the end, before reusing the ring
            asm volatile("" ::: "memory");
            finish_v(acc);
        }
        wait_vmcnt<0>();
        asm volatile("" ::: "memory");
    } else {
        // ========================= BF16 ring chunks (binary32) =========================
        // units of 32 tokens; a step is two halves of 16 tokens (8 lanes per token pair)
        const int R = g.ring_slots;
        if (kwave) {
            float mh = kNeg;                           // running max of the lane's head kb
            float lsum = 0.0f;                         // sum of p of the lane's head
            float qr[kG][16];
#pragma unroll
            for (int h = 0; h < kG; ++h)
#pragma unroll
                for (int j = 0; j < 16; ++j) qr[h][j] = S.qs[h][16 * vp + j];
            int j = 0;
#pragma unroll 1
            for (; j < J; ++j) {
                const int64_t tb = sq.n_q + (int64_t)(u_first + 2 * j) * kTailUnit;
                const int64_t te = min<int64_t>(tb + kTailUnit, sq.n);
                const uint32_t tbm = (uint32_t)(tb % R);
                float sc[2][kG][2];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int off = 16 * half + 2 * vg;
                    uint4 w[2][2];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int o = min<int64_t>(off + t, te - tb - 1);
                        const uint32_t rs = (tbm + (uint32_t)o) % (uint32_t)R;
                        const uint4* pk = (const uint4*)(kst + g.k.ring + (int64_t)rs * 256 + 32 * vp);
                        w[t][0] = pk[0];
                        w[t][1] = pk[1];
                    }
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const uint32_t ww[8] = {w[t][0].x, w[t][0].y, w[t][0].z, w[t][0].w,
                                                w[t][1].x, w[t][1].y, w[t][1].z, w[t][1].w};
                        float kx[16];
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            kx[2 * i] = bf16_to_f32(ww[i] & 0xFFFFu);
                            kx[2 * i + 1] = bf16_to_f32(ww[i] >> 16);
                        }
#pragma unroll
                        for (int h = 0; h < kG; ++h) {
                            float x = 0.0f;
#pragma unroll
                            for (int jj = 0; jj < 16; ++jj) x = fmaf(qr[h][jj], kx[jj], x);
                            x += dpp<QP_XOR1>(x);
                            x += dpp<QP_XOR2>(x);
                            x += dpp<ROW_HMIRROR>(x);
                            sc[half][h][t] = (tb + off + t < te) ? x : kNeg;
                        }
                    }
                }
                // each lane keeps the scores of head vp & 3; lanes with equal vp share a head
                const int hv = vp & 3;
                float x[2][2];
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const f32x4 v = {sc[half][0][t], sc[half][1][t], sc[half][2][t], sc[half][3][t]};
                        x[half][t] = v[hv];
                    }
                const float nm = fmaxf(mh, wave_max8(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[1][0], x[1][1]))));
                const float al = __builtin_amdgcn_exp2f(mh - nm);    // exactly 1 if unchanged
                mh = nm;
                lsum *= al;
                PBuf& P = S.pb[pr][j & 1];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int off = 16 * half + 2 * vg;
                    const float p0 = (tb + off < te) ? __builtin_amdgcn_exp2f(x[half][0] - mh) : 0.0f;
                    const float p1 = (tb + off + 1 < te) ? __builtin_amdgcn_exp2f(x[half][1] - mh) : 0.0f;
                    if (vp < kG) {
                        *(float2*)&P.p[8 * half + vg][vp][0] = make_float2(p0, p1);
                        lsum += p0 + p1;
                    }
                }
                if (lane < kG) P.alpha[lane] = al;
                __syncthreads();
            }
#pragma unroll 1
            for (; j <= Jmax; ++j) __syncthreads();
            finish_k(mh, lsum, false);
        } else {
            float acc[kG][16];
#pragma unroll
            for (int h = 0; h < kG; ++h)
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) acc[h][jj] = 0.0f;
            __syncthreads();
            int j = 0;
#pragma unroll 1
            for (; j < J; ++j) {
                const int64_t tb = sq.n_q + (int64_t)(u_first + 2 * j) * kTailUnit;
                const int64_t te = min<int64_t>(tb + kTailUnit, sq.n);
                const uint32_t tbm = (uint32_t)(tb % R);
                const PBuf& P = S.pb[pr][j & 1];
                const float4 al = *(const float4*)P.alpha;
                if (al.x != 1.0f || al.y != 1.0f || al.z != 1.0f || al.w != 1.0f) {
                    const float alv[kG] = {al.x, al.y, al.z, al.w};
#pragma unroll
                    for (int h = 0; h < kG; ++h)
#pragma unroll
                        for (int jj = 0; jj < 16; ++jj) acc[h][jj] *= alv[h];
                }
#pragma unroll 1
                for (int half = 0; half < 2; ++half) {
                    const int slot = vg + 8 * half;
                    const int off = 2 * slot;
                    float vx[2][16];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int o = min<int64_t>(off + t, te - tb - 1);
                        const uint32_t rs = (tbm + (uint32_t)o) % (uint32_t)R;
                        const uint4* pv = (const uint4*)(vst + g.v.ring + (int64_t)rs * 256 + 32 * vp);
                        const uint4 w0 = pv[0], w1 = pv[1];
                        const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            vx[t][2 * i] = bf16_to_f32(ww[i] & 0xFFFFu);
                            vx[t][2 * i + 1] = bf16_to_f32(ww[i] >> 16);
                        }
                    }
                    const float4 pa = *(const float4*)&P.p[slot][0][0];
                    const float4 pb = *(const float4*)&P.p[slot][2][0];
                    const float pp[4][2] = {{pa.x, pa.y}, {pa.z, pa.w}, {pb.x, pb.y}, {pb.z, pb.w}};
#pragma unroll
                    for (int h = 0; h < kG; ++h)
#pragma unroll
                        for (int jj = 0; jj < 16; ++jj)
                            acc[h][jj] = fmaf(pp[h][0], vx[0][jj], fmaf(pp[h][1], vx[1][jj], acc[h][jj]));
                }
                __syncthreads();
            }
#pragma unroll 1
            for (++j; j <= Jmax; ++j) __syncthreads();
            finish_v(acc);
        }
    }

    __syncthreads();
    float* part_out = a.partials + (int64_t)bid * kPartialFloats;
    for (int i = tid; i < kG * kD; i += blockDim.x) {
        const int h = i / kD, d = i % kD;
        const float M = fmaxf(S.wm[0][h], S.wm[1][h]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const float ew = __builtin_amdgcn_exp2f(S.wm[p][h] - M);
            L += S.wl[p][h] * ew;
            A += reinterpret_cast<const float (*)[kD]>(&S.st[2 + p][0])[h][d] * ew;
        }
        part_out[2 * kMaxGroup + h * kD + d] = A;
        if (d == 0) { part_out[h] = M; part_out[kMaxGroup + h] = L; }
    }
}

template <int FMT>
int launch_ws_fmt(const DecodeArgs& a, int n_wgs, hipStream_t st)
{
    hipLaunchKernelGGL(k_decode_ws<FMT>, dim3(n_wgs), dim3(256), 0, st, a);
    return (int)hipGetLastError();
}

template <int FMT>
int occ_ws()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_decode_ws<FMT>, 256, 0) != hipSuccess) return 0;
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
    case 5: return launch_ws_fmt<5>(a, n_wgs, st);
    case 6: return launch_ws_fmt<6>(a, n_wgs, st);
    case 15: return launch_ws_fmt<15>(a, n_wgs, st);
    default: return (int)hipErrorInvalidValue;
    }
}

int decode_fast_wgs_per_cu(int fmt)
{
    static int cache[19] = {0};
    if (fmt < 0 || fmt >= 19) return 0;
    if (!cache[fmt]) {
        switch (fmt) {
        case 5: cache[fmt] = occ_ws<5>(); break;
        case 6: cache[fmt] = occ_ws<6>(); break;
        case 15: cache[fmt] = occ_ws<15>(); break;
        default: return 0;
        }
    }
    return cache[fmt];
}

}  // namespace kvq
