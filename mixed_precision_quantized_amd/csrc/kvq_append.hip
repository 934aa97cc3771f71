// kvq_append.hip -- quantize-on-append kernels for gfx950.
//
//  * k_encode_q<FMT>: qN_0 / qN_1 / bf16 encoding of whole tokens (4 lanes per token and
//    stream, one 32-dim block per lane).  Symmetric qN_0 takes its fp16 scale from the
//    signed max-magnitude element and uses all 2^N levels; qN_1 stores an fp16 step
//    (max-min)/(2^N-1) and an fp16 min.  Codes are a little-endian N-bit stream per token.
//  * k_kvarn_page<N>: KVarN for one 128-token page of one stream per workgroup: unnormalized
//    Walsh-Hadamard rotation of every token vector, 8 Sinkhorn iterations balancing
//    per-token and per-channel mean squares, fp16 channel scales, then qN_0 (kvarnN) or
//    qN_1 (kvarnN_1, AFF) of the normalized values ("Практическое руководство: запуск Bonsai-Ternary-27B на 120k
//    токенах с менее чем 10 ГБ VRAM", sections "Решение: KVarN ..." and "Как
//    преобразование Уолша-Адамара и Sinkhorn спасают качество при 4-битном сжатии").
//  * k_ring_write: canonical 16-bit rows of the newest tokens into the precision-tail ring.
//
// Every value is the canonical 16-bit form of the input, bf16 or (F16 tail) binary16, both
// rounded to nearest even, so codes depend only on a token's (or its page's) values, never
// on when it is spilled.
#pragma clang fp contract(off)

#include <float.h>

#include "kvq_device.h"

namespace kvq {

namespace {

__device__ __forceinline__ char* stream_ptr(const CacheGeom& g, int seq, int layer, int head, int isv)
{
    int64_t unit = ((int64_t)seq * g.n_layers + layer) * g.n_kv_heads + head;
    return g.base + unit * g.unit_bytes + (isv ? g.v_offset : 0);
}

// Address of the 128 input values of (layer - layer0, row, head) for K (isv=0) or V.
__device__ __forceinline__ const char* input_row(const AppendArgs& a, int lrel, int64_t row, int head, int isv)
{
    const char* base = (const char*)(isv ? a.v_in : a.k_in);
    int64_t elem = (((int64_t)lrel * a.rows + row) * a.g.n_kv_heads + head) * kD;
    return base + elem * (a.in_dtype ? 4 : 2);
}

// Load NV consecutive canonical values (as floats) starting at element e0 of a row that is
// a ring row (canonical already), an fp32 input row or a bf16 input row (both rounded to
// the canonical type first; a bf16 input is its own canonical value for a BF16 tail).
template <int NV, bool f16>
__device__ __forceinline__ void load_canon_t(const char* row, bool f32, bool ring, int e0, float (&x)[NV])
{
    if (f32) {
        const float4* p = (const float4*)(row + 4 * e0);
#pragma unroll
        for (int i = 0; i < NV / 4; ++i) {
            float4 w = p[i];
            x[4 * i + 0] = canon_to_f32(canon_bits(w.x, f16), f16);
            x[4 * i + 1] = canon_to_f32(canon_bits(w.y, f16), f16);
            x[4 * i + 2] = canon_to_f32(canon_bits(w.z, f16), f16);
            x[4 * i + 3] = canon_to_f32(canon_bits(w.w, f16), f16);
        }
    } else {
        const uint4* p = (const uint4*)(row + 2 * e0);
        // ring rows hold the canonical type; bf16 input rows are rounded to binary16 for F16
        const bool conv = f16 && !ring;
        auto val = [&](uint32_t h) {
            return conv ? canon_to_f32(canon_bits(bf16_to_f32(h), true), true) : canon_to_f32(h, f16 && ring);
        };
#pragma unroll
        for (int i = 0; i < NV / 8; ++i) {
            uint4 w = p[i];
            x[8 * i + 0] = val(w.x & 0xFFFFu);
            x[8 * i + 1] = val(w.x >> 16);
            x[8 * i + 2] = val(w.y & 0xFFFFu);
            x[8 * i + 3] = val(w.y >> 16);
            x[8 * i + 4] = val(w.z & 0xFFFFu);
            x[8 * i + 5] = val(w.z >> 16);
            x[8 * i + 6] = val(w.w & 0xFFFFu);
            x[8 * i + 7] = val(w.w >> 16);
        }
    }
}
// the canonical type chosen once per call (a uniform branch), not per value
template <int NV>
__device__ __forceinline__ void load_canon(const char* row, bool f32, bool ring, bool f16, int e0, float (&x)[NV])
{
    if (f16) load_canon_t<NV, true>(row, f32, ring, e0, x);
    else load_canon_t<NV, false>(row, f32, ring, e0, x);
}

// clamp(rint(t) + off, 0, top) in binary32, rint = round half to even.
// (max/min give the same codes as the comparisons: v is never NaN, and -0 converts to 0.)
__device__ __forceinline__ uint32_t code_of(float t, float off, float top)
{
    const float v = __builtin_rintf(t) + off;
    return (uint32_t)__builtin_fminf(__builtin_fmaxf(v, 0.0f), top);
}

// Pack 32 N-bit codes into N little-endian 32-bit words.
template <int N>
__device__ __forceinline__ void pack32(const uint32_t (&u)[32], uint32_t (&w)[N])
{
#pragma unroll
    for (int k = 0; k < N; ++k) w[k] = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int bit = i * N;
        const int wi = bit >> 5, sh = bit & 31;
        w[wi] |= u[i] << sh;
        if (sh + N > 32) w[wi + 1] |= u[i] >> (32 - sh);
    }
}

// Largest and smallest of a block.  The inputs are finite (no NaN), so the hardware
// max/min give the same values as a scan with strict comparisons, except possibly for the
// sign of a zero extreme, which changes no scale and no code: a zero signed maximum gives
// d = fp16(+-0) = +0 (all codes at the offset), a zero range gives step +0, and the stored
// minimum is fp16(+-0) = +0 either way.
__device__ __forceinline__ void block_max_min(const float (&x)[32], float& mx, float& mn)
{
    float a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = __builtin_fmaxf(__builtin_fmaxf(x[i], x[i + 8]), __builtin_fmaxf(x[i + 16], x[i + 24]));
        b[i] = __builtin_fminf(__builtin_fminf(x[i], x[i + 8]), __builtin_fminf(x[i + 16], x[i + 24]));
    }
#pragma unroll
    for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) {
            a[i] = __builtin_fmaxf(a[i], a[i + w]);
            b[i] = __builtin_fminf(b[i], b[i + w]);
        }
    mx = a[0];
    mn = b[0];
}

// Symmetric block encoder: returns the fp16 scale bits, fills 32 codes.
template <int N>
__device__ __forceinline__ uint32_t encode_block_q0(const float (&x)[32], uint32_t (&u)[32])
{
    float mx, mn;
    block_max_min(x, mx, mn);
    const float m = (mx >= -mn) ? mx : mn;
    const float qd = m / -(float)(1 << (N - 1));
    const uint32_t d = fp16s_rne(qd);
    if (d == 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i) u[i] = 1u << (N - 1);
        return 0;
    }
    const float inv = 1.0f / fp16_to_f32(d);
    const float off = (float)(1 << (N - 1)), top = (float)((1 << N) - 1);
#pragma unroll
    for (int i = 0; i < 32; ++i) u[i] = code_of(x[i] * inv, off, top);
    return d;
}

// Affine block encoder: returns d | m << 16, fills 32 codes.
template <int N>
__device__ __forceinline__ uint32_t encode_block_q1(const float (&x)[32], uint32_t (&u)[32])
{
    float mx, mn;
    block_max_min(x, mx, mn);
    const float top = (float)((1 << N) - 1);
    const float dr = mx - mn;
    const float dq = dr / top;
    const uint32_t d = fp16s_rne(dq);
    const uint32_t m = fp16s_rne(mn);
    if (d == 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i) u[i] = 0;
        return m << 16;
    }
    const float mf = fp16_to_f32(m);
    const float inv = 1.0f / fp16_to_f32(d);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        float diff = x[i] - mf;
        u[i] = code_of(diff * inv, 0.0f, top);
    }
    return d | (m << 16);
}

template <int N>
__device__ __forceinline__ void store_words(char* dst, const uint32_t (&w)[N])
{
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int k = 0; k < N; k += 4) *(uint4*)(dst + 4 * k) = make_uint4(w[k], w[k + 1], w[k + 2], w[k + 3]);
    } else if constexpr (N % 2 == 0) {
#pragma unroll
        for (int k = 0; k < N; k += 2) *(uint2*)(dst + 4 * k) = make_uint2(w[k], w[k + 1]);
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) *(uint32_t*)(dst + 4 * k) = w[k];
    }
}

// Locate the sequence entry of a token index t in [0, total) where entry i owns
// count_i consecutive indices; returns the entry and the offset inside it.
template <typename CountFn>
__device__ __forceinline__ int find_entry(const AppendArgs& a, int64_t t, int64_t* off, CountFn cnt)
{
    int64_t acc = 0;
    for (int i = 0; i < a.n_seqs; ++i) {
        int64_t c = cnt(a.seqs[i]);
        if (t < acc + c) { *off = t - acc; return i; }
        acc += c;
    }
    *off = 0;
    return -1;
}

struct EncCount { __device__ int64_t operator()(const AppendSeq& s) const { return s.nq_new - s.nq_old; } };
struct RingCount {
    __device__ int64_t operator()(const AppendSeq& s) const
    {
        int64_t lo = s.nq_new > s.n_old ? s.nq_new : s.n_old;
        return s.n_new > lo ? s.n_new - lo : 0;
    }
};
struct PageCount { __device__ int64_t operator()(const AppendSeq& s) const { return (s.nq_new - s.nq_old) / kPage; } };

// ------------------------------------------------------------------ qN / bf16 encoder
// Lane work item: (layer, head, stream, token, block), token-fastest within a stream.
// sv_sel: 0 or 1 encodes only the K or the V stream (their formats differ), 2 both.
template <int FMT>
__global__ __launch_bounds__(256) void k_encode_q(AppendArgs a, int64_t tokens, int sv_sel)
{
    constexpr int N = fbits(FMT);
    constexpr int KIND = fkind(FMT);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int b = (int)(gid & 3);
    int64_t w = gid >> 2;
    const int64_t tg = w % tokens;
    w /= tokens;
    int sv = sv_sel;
    if (sv_sel == 2) {
        sv = (int)(w & 1);
        w >>= 1;
    }
    const int head = (int)(w % a.g.n_kv_heads);
    const int lrel = (int)(w / a.g.n_kv_heads);
    if (lrel >= a.layers_in) return;
    int64_t off;
    const int e = find_entry(a, tg, &off, EncCount());
    if (e < 0) return;
    const AppendSeq& s = a.seqs[e];
    const int64_t p = s.nq_old + off;
    const int layer = a.layer0 + lrel;
    char* st = stream_ptr(a.g, s.seq, layer, head, sv);
    const StreamLayout& L = sv ? a.g.v : a.g.k;
    const bool from_ring = p < s.n_old;
    const char* src = from_ring ? st + L.ring + (p % a.g.ring_slots) * 256
                                : input_row(a, lrel, s.in_row0 + (p - s.n_old), head, sv);
    const bool f32 = !from_ring && a.in_dtype == 1;
    char* codes = st + L.codes + p * fcode_bytes(FMT);

    if constexpr (KIND == KIND_BF16) {
        // identity: the canonical bf16 row
        uint32_t o[16];
        if (f32) {
            const float4* q = (const float4*)(src + 4 * 32 * b);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float4 v = q[i];
                o[2 * i] = bf16_rne(v.x) | ((uint32_t)bf16_rne(v.y) << 16);
                o[2 * i + 1] = bf16_rne(v.z) | ((uint32_t)bf16_rne(v.w) << 16);
            }
        } else {
            const uint4* q = (const uint4*)(src + 2 * 32 * b);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint4 v = q[i];
                o[4 * i] = v.x; o[4 * i + 1] = v.y; o[4 * i + 2] = v.z; o[4 * i + 3] = v.w;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *(uint4*)(codes + 64 * b + 16 * i) = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    } else {
        float x[32];
        load_canon<32>(src, f32, from_ring, a.g.tail_f16 != 0, 32 * b, x);
        uint32_t u[32];
        uint32_t packed[N];
        char* scales = st + L.scales + p * (fscale_halves(FMT) * 2);
        if constexpr (KIND == KIND_Q0) {
            uint32_t d = encode_block_q0<N>(x, u);
            *(uint16_t*)(scales + 2 * b) = (uint16_t)d;
        } else {
            uint32_t dm = encode_block_q1<N>(x, u);
            *(uint32_t*)(scales + 4 * b) = dm;
        }
        pack32<N>(u, packed);
        store_words<N>(codes + 4 * N * b, packed);
    }
}

// ------------------------------------------------------------------ ring writer
// 8 lanes per (token, stream), 16 values per lane.
__global__ __launch_bounds__(256) void k_ring_write(AppendArgs a, int64_t tokens)
{
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int part = (int)(gid & 7);
    int64_t w = gid >> 3;
    const int64_t tg = w % tokens;
    w /= tokens;
    const int sv = (int)(w & 1);
    w >>= 1;
    const int head = (int)(w % a.g.n_kv_heads);
    const int lrel = (int)(w / a.g.n_kv_heads);
    if (lrel >= a.layers_in) return;
    int64_t off;
    const int e = find_entry(a, tg, &off, RingCount());
    if (e < 0) return;
    const AppendSeq& s = a.seqs[e];
    const int64_t lo = s.nq_new > s.n_old ? s.nq_new : s.n_old;
    const int64_t p = lo + off;
    const int layer = a.layer0 + lrel;
    char* st = stream_ptr(a.g, s.seq, layer, head, sv);
    const StreamLayout& L = sv ? a.g.v : a.g.k;
    const char* src = input_row(a, lrel, s.in_row0 + (p - s.n_old), head, sv);
    char* dst = st + L.ring + (p % a.g.ring_slots) * 256 + 32 * part;
    const bool f16 = a.g.tail_f16 != 0;
    if (a.in_dtype == 1) {
        const float4* q = (const float4*)(src + 64 * part);
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 v = q[i];
            o[2 * i] = canon_bits(v.x, f16) | (canon_bits(v.y, f16) << 16);
            o[2 * i + 1] = canon_bits(v.z, f16) | (canon_bits(v.w, f16) << 16);
        }
        *(uint4*)dst = make_uint4(o[0], o[1], o[2], o[3]);
        *(uint4*)(dst + 16) = make_uint4(o[4], o[5], o[6], o[7]);
    } else if (f16) {
        // bf16 input, binary16 ring
        const uint4* q = (const uint4*)(src + 32 * part);
        const uint4 w0 = q[0], w1 = q[1];
        const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i] = canon_bits(bf16_to_f32(w[i] & 0xFFFFu), true) | (canon_bits(bf16_to_f32(w[i] >> 16), true) << 16);
        *(uint4*)dst = make_uint4(o[0], o[1], o[2], o[3]);
        *(uint4*)(dst + 16) = make_uint4(o[4], o[5], o[6], o[7]);
    } else {
        const uint4* q = (const uint4*)(src + 32 * part);
        *(uint4*)dst = q[0];
        *(uint4*)(dst + 16) = q[1];
    }
}

// ------------------------------------------------------------------ KVarN page encoder
// One 128 x 128 page of one stream per workgroup of 256 threads.
//
// Phases: (1) thread (t, half) loads half of token row t and rotates the row (six
// butterfly stages in registers, the last across the lane pair); the rotated values y stay
// in its registers until the encode.  (2) The squares A = y^2 move through LDS, half a page
// at a time, into the register tile of the Sinkhorn layout: thread (r0, c0) holds
// A[r0 + 16 k][c0 + 16 m], k, m = 0..7 (r0, c0 = the low 4 bits of token and channel).
// (3) Every Sinkhorn sum adds 128 products in the halving-tree order (index bit 6 first,
// bit 0 last): bits 6..4 are the k or m of the tile, in registers; the row sums' bits 3..0
// are c0, the lane bits 0..3, combined by DPP (lane ^ 8, ^ 4, ^ 2, ^ 1, every lane
// ending with the total); the column sums' bits 3..0 are r0, which spans the four waves,
// so the partials go through LDS and 128 threads finish one column each.  Each reciprocal
// is taken once (one row per lane of a 16-lane row, then broadcast; one column per
// thread).  (4) fp16 channel scales, (5) normalize and block-encode the thread's own
// half-row, pack, store.
constexpr int kRedStride = 144;   // row of the column partials (rows 16 words apart in the banks)

// XOR swizzle of the transposition buffer [64][128]: column j of token row tl (0..63) sits
// at word tl * 128 + (j ^ swz(tl, j >> 6)).  Bank conflict free both for the row writes
// (lanes = 32 tokens x 2 halves) and for the tile reads (lanes = 16 channels x 4 tokens).
__device__ __forceinline__ int swz(int tl, int h)
{
    const int b0 = (tl >> 2) & 1, b1 = (tl >> 3) & 1, b2 = ((tl >> 4) ^ (tl >> 1)) & 1;
    return b0 | (b1 << 1) | (b2 << 2) | (h << 3) | ((tl & 1) << 4) | (((tl >> 1) & 1) << 5);
}

__device__ __forceinline__ float swap_pair(float x)
{
    // exchange with the neighbouring lane (lanes 2k <-> 2k+1): DPP quad_perm [1,0,3,2]
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ float dppf(float x)
{
    // every lane reads a valid lane in these patterns; bound_ctrl lets the compiler fold
    // the move into the add that uses it
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// within each row of 16 lanes: lane ^ 8 (rotate by 8), lane ^ 2, lane ^ 1 (quad
// permutes); rotate by 4 stands for lane ^ 4 once lanes l and l ^ 8 hold equal values
constexpr int kRor8 = 0x128, kRor4 = 0x124, kXor2 = 0x4E, kXor1 = 0xB1;
constexpr int kNewBcast0 = 0x150;   // row_newbcast:n, lane n of the row to the whole row

template <int N, bool AFF>
__global__ __launch_bounds__(256) void k_kvarn_page(AppendArgs a, int64_t pages, int streams_mask)
{
    __shared__ float tr[64 * kD];              // squares of half a page, swizzled
    __shared__ float red[16 * kRedStride];     // column partials [r0][channel]
    __shared__ float ic_s[kPage];              // 1 / c2 of the last column step
    __shared__ float c2_s[kPage];              // c2 of the last iteration
    __shared__ float ic16_s[kPage];            // 1 / fp16 channel scale

    const int tid = threadIdx.x;
    int64_t w = blockIdx.x;
    const int64_t pg = w % pages;
    w /= pages;
    const int sv = (int)(w & 1);
    w >>= 1;
    const int head = (int)(w % a.g.n_kv_heads);
    const int lrel = (int)(w / a.g.n_kv_heads);
    if (!((streams_mask >> sv) & 1)) return;
    int64_t off;
    const int e = find_entry(a, pg, &off, PageCount());
    if (e < 0) return;
    const AppendSeq& s = a.seqs[e];
    const int64_t page = s.nq_old / kPage + off;
    const int layer = a.layer0 + lrel;
    char* st = stream_ptr(a.g, s.seq, layer, head, sv);
    const StreamLayout& L = sv ? a.g.v : a.g.k;

    // ---- 1. load half a token row (64 values) and rotate it --------------------------
    const int t = tid >> 1;            // token of the page
    const int half = tid & 1;          // dims [64*half, 64*half+64)
    const int64_t p = page * kPage + t;
    const bool from_ring = p < s.n_old;
    const char* src = from_ring ? st + L.ring + (p % a.g.ring_slots) * 256
                                : input_row(a, lrel, s.in_row0 + (p - s.n_old), head, sv);
    float y[64];
    load_canon<64>(src, !from_ring && a.in_dtype == 1, from_ring, a.g.tail_f16 != 0, 64 * half, y);
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            if (i & h) continue;
            float u = y[i], v = y[i + h];
            y[i] = u + v;
            y[i + h] = u - v;
        }
    }
    // stage h = 64 pairs dim i with i+64: the other half lives in the neighbouring lane
    // (y sg + o with sg = +-1 is y + o or o - y exactly: the product is exact, so the fused
    // form rounds once, like the sum)
    const float sg = half ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) y[i] = __builtin_fmaf(y[i], sg, swap_pair(y[i]));

    // ---- 2. squares into the Sinkhorn tile, through LDS half a page at a time -----------
    const int lane = tid & 63;
    const int c0 = lane & 15;
    const int r0 = (lane >> 4) | ((tid >> 6) << 2);
    float A[8][8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        if ((t >> 6) == hh) {
            const int tl = t & 63;
            const int sw = swz(tl, half);
#pragma unroll
            for (int i = 0; i < 64; ++i) tr[tl * kD + ((64 * half + i) ^ sw)] = y[i] * y[i];
        }
        __syncthreads();
#pragma unroll
        for (int k = 4 * hh; k < 4 * hh + 4; ++k) {
            const int tl = r0 + 16 * (k & 3);
#pragma unroll
            for (int m = 0; m < 8; ++m) A[k][m] = tr[tl * kD + ((c0 + 16 * m) ^ swz(tl, m >> 2))];
        }
        __syncthreads();
    }

    // ---- 3. Sinkhorn: 8 x (row step, column step) ---------------------------------------
    const float inv128 = 1.0f / 128.0f;
    float ic[8];                       // 1 / c2 of the thread's channels c0 + 16 m
#pragma unroll
    for (int m = 0; m < 8; ++m) ic[m] = 1.0f;
    for (int it = 0; it < 8; ++it) {
        // row step: r2[t] = (sum_j A[t][j] / c2[j]) / 128
        float rs[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float v[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) v[m] = A[k][m] * ic[m];
#pragma unroll
            for (int m = 0; m < 4; ++m) v[m] = v[m] + v[m + 4];
            v[0] = v[0] + v[2];
            v[1] = v[1] + v[3];
            float x = v[0] + v[1];
            x = x + dppf<kRor8>(x);
            x = x + dppf<kRor4>(x);
            x = x + dppf<kXor2>(x);
            x = x + dppf<kXor1>(x);
            rs[k] = x;
        }
        // lane c0 of each 16-lane row takes the reciprocal of row k = c0 & 7 (the others
        // repeat it); the row then gets every lane's value back by broadcast
        float sel = rs[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) sel = (c0 & 7) == k ? rs[k] : sel;
        float r = sel * inv128;
        if (!(r >= FLT_MIN)) r = 1.0f;
        const float irs = 1.0f / r;
        float ir[8];
        ir[0] = dppf<kNewBcast0 + 0>(irs);
        ir[1] = dppf<kNewBcast0 + 1>(irs);
        ir[2] = dppf<kNewBcast0 + 2>(irs);
        ir[3] = dppf<kNewBcast0 + 3>(irs);
        ir[4] = dppf<kNewBcast0 + 4>(irs);
        ir[5] = dppf<kNewBcast0 + 5>(irs);
        ir[6] = dppf<kNewBcast0 + 6>(irs);
        ir[7] = dppf<kNewBcast0 + 7>(irs);
        // column step: c2[j] = (sum_t A[t][j] / r2[t]) / 128; the tile's part (token bits
        // 6..4), then bits 3..0 (r0) by the column's thread
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = A[k][m] * ir[k];
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = v[k] + v[k + 4];
            v[0] = v[0] + v[2];
            v[1] = v[1] + v[3];
            red[r0 * kRedStride + c0 + 16 * m] = v[0] + v[1];
        }
        __syncthreads();
        if (tid < kPage) {
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = red[i * kRedStride + tid];
#pragma unroll
            for (int wd = 8; wd >= 1; wd >>= 1) {
#pragma unroll
                for (int i = 0; i < wd; ++i) v[i] = v[i] + v[i + wd];
            }
            float c = v[0] * inv128;
            if (!(c >= FLT_MIN)) c = 1.0f;
            ic_s[tid] = 1.0f / c;
            c2_s[tid] = c;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 8; ++m) ic[m] = ic_s[c0 + 16 * m];
    }
    // ---- 4. channel scales ----------------------------------------------------------
    if (tid < kPage) {
        uint32_t c = fp16s_rne(__builtin_sqrtf(c2_s[tid]));
        if (c == 0) c = 0x3C00u;
        ic16_s[tid] = 1.0f / fp16_to_f32(c);
        ((uint16_t*)(st + L.cscale + page * 256))[tid] = (uint16_t)c;
    }
    __syncthreads();
    // ---- 5./6. normalize, block quantization (symmetric or affine), pack ------------------
    char* codes = st + L.codes + p * (16 * N);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        float x[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = y[32 * bb + i] * ic16_s[64 * half + 32 * bb + i];
        uint32_t u[32];
        const uint32_t d = AFF ? encode_block_q1<N>(x, u) : encode_block_q0<N>(x, u);
        uint32_t packed[N];
        pack32<N>(u, packed);
        const int blk = 2 * half + bb;
        store_words<N>(codes + 4 * N * blk, packed);
        if (AFF) ((uint32_t*)(st + L.scales + p * 16))[blk] = d;   // step | minimum << 16
        else ((uint16_t*)(st + L.scales + p * 8))[blk] = (uint16_t)d;
    }
}

inline int64_t total_of(const AppendArgs& a, int which)
{
    int64_t tot = 0;
    for (int i = 0; i < a.n_seqs; ++i) {
        const AppendSeq& s = a.seqs[i];
        if (which == 0) tot += s.nq_new - s.nq_old;
        else if (which == 1) {
            int64_t lo = s.nq_new > s.n_old ? s.nq_new : s.n_old;
            tot += s.n_new > lo ? s.n_new - lo : 0;
        } else {
            tot += (s.nq_new - s.nq_old) / kPage;
        }
    }
    return tot;
}

template <int FMT>
int launch_enc(const AppendArgs& a, int64_t tokens, int sv_sel, hipStream_t st)
{
    int64_t lanes = 4 * tokens * (sv_sel == 2 ? 2 : 1) * a.g.n_kv_heads * (int64_t)a.layers_in;
    int64_t blocks = (lanes + 255) / 256;
    hipLaunchKernelGGL(k_encode_q<FMT>, dim3((unsigned)blocks), dim3(256), 0, st, a, tokens, sv_sel);
    return (int)hipGetLastError();
}

int launch_enc_fmt(int fmt, const AppendArgs& a, int64_t tokens, int sv_sel, hipStream_t st)
{
    switch (fmt) {
    case 0: return launch_enc<0>(a, tokens, sv_sel, st);
    case 1: return launch_enc<1>(a, tokens, sv_sel, st);
    case 2: return launch_enc<2>(a, tokens, sv_sel, st);
    case 3: return launch_enc<3>(a, tokens, sv_sel, st);
    case 4: return launch_enc<4>(a, tokens, sv_sel, st);
    case 5: return launch_enc<5>(a, tokens, sv_sel, st);
    case 6: return launch_enc<6>(a, tokens, sv_sel, st);
    case 7: return launch_enc<7>(a, tokens, sv_sel, st);
    case 8: return launch_enc<8>(a, tokens, sv_sel, st);
    case 9: return launch_enc<9>(a, tokens, sv_sel, st);
    case 10: return launch_enc<10>(a, tokens, sv_sel, st);
    case 11: return launch_enc<11>(a, tokens, sv_sel, st);
    case 12: return launch_enc<12>(a, tokens, sv_sel, st);
    default: return (int)hipErrorInvalidValue;
    }
}

template <int N, bool AFF>
int launch_kv(const AppendArgs& a, int64_t pages, int mask, hipStream_t st)
{
    int64_t blocks = pages * 2 * a.g.n_kv_heads * (int64_t)a.layers_in;
    hipLaunchKernelGGL((k_kvarn_page<N, AFF>), dim3((unsigned)blocks), dim3(256), 0, st, a, pages, mask);
    return (int)hipGetLastError();
}

}  // namespace

int launch_append_encode(const AppendArgs& a, void* stream)
{
    int64_t tokens = total_of(a, 0);
    if (tokens <= 0) return 0;
    hipStream_t st = (hipStream_t)stream;
    // token-wise formats only; a KVarN stream is encoded page-wise (launch_append_kvarn)
    const bool kq = !kind_paged(fkind(a.g.fmt_k)), vq = !kind_paged(fkind(a.g.fmt_v));
    if (kq && vq && a.g.fmt_k == a.g.fmt_v) return launch_enc_fmt(a.g.fmt_k, a, tokens, 2, st);
    int rc = 0;
    if (kq) rc = launch_enc_fmt(a.g.fmt_k, a, tokens, 0, st);
    if (!rc && vq) rc = launch_enc_fmt(a.g.fmt_v, a, tokens, 1, st);
    return rc;
}

int launch_append_kvarn(const AppendArgs& a, void* stream)
{
    int64_t pages = total_of(a, 2);
    if (pages <= 0) return 0;
    hipStream_t st = (hipStream_t)stream;
    // one launch per format: mask bit 0 = K stream, bit 1 = V stream
    auto launch_n = [&](int fmt, int mask) -> int {
        const bool aff = fkind(fmt) == KIND_KVARN1;
        switch (fbits(fmt)) {
        case 2: return aff ? launch_kv<2, true>(a, pages, mask, st) : launch_kv<2, false>(a, pages, mask, st);
        case 3: return aff ? launch_kv<3, true>(a, pages, mask, st) : launch_kv<3, false>(a, pages, mask, st);
        case 4: return aff ? launch_kv<4, true>(a, pages, mask, st) : launch_kv<4, false>(a, pages, mask, st);
        case 5: return aff ? launch_kv<5, true>(a, pages, mask, st) : launch_kv<5, false>(a, pages, mask, st);
        case 6: return aff ? launch_kv<6, true>(a, pages, mask, st) : launch_kv<6, false>(a, pages, mask, st);
        case 8: return aff ? launch_kv<8, true>(a, pages, mask, st) : launch_kv<8, false>(a, pages, mask, st);
        default: return (int)hipErrorInvalidValue;
        }
    };
    const bool kk = kind_paged(fkind(a.g.fmt_k)), vk = kind_paged(fkind(a.g.fmt_v));
    if (kk && vk && a.g.fmt_k == a.g.fmt_v) return launch_n(a.g.fmt_k, 3);
    int rc = 0;
    if (kk) rc = launch_n(a.g.fmt_k, 1);
    if (!rc && vk) rc = launch_n(a.g.fmt_v, 2);
    return rc;
}

int launch_append_ring(const AppendArgs& a, void* stream)
{
    int64_t tokens = total_of(a, 1);
    if (tokens <= 0) return 0;
    int64_t lanes = 8 * tokens * 2 * a.g.n_kv_heads * (int64_t)a.layers_in;
    int64_t blocks = (lanes + 255) / 256;
    hipLaunchKernelGGL(k_ring_write, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a, tokens);
    return (int)hipGetLastError();
}

}  // namespace kvq
