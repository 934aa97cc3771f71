// kvq_decode_ws.h -- fast decode attention for quantized caches of 2- to 6- and 8-bit codes
// (qN_0, qN_1, kvarnN, kvarnN_1), gfx950.  The kernel template; kvq_decode_ws_key.hip
// instantiates one key format against every value format per translation unit.
//
// Same work split as the generic kernel (kvq_decode.hip): 128-token quantized pages and
// 32-token ring chunks, balanced splits, partial results merged by kvq_merge.hip.  One
// workgroup of 16 waves per CU; inside it the waves specialize, so each role fits in 128
// VGPRs and four waves share every SIMD:
//
//   "K waves"  score 32 tokens per step and run the online softmax;
//   "V waves"  accumulate the values of the step the K waves finished before.
//
// A K wave and a V wave form a pair; the 8 pairs of a workgroup walk interleaved pages and
// hand the probabilities of a step over through LDS, and the whole workgroup takes one
// barrier per step, which keeps all 16 waves in lockstep (separate smaller workgroups
// drift apart: the oldest wins instruction issue).  In each group of four waves the K
// waves sit on SIMDs 0, 1 or 2, 3 alternately, so every SIMD runs both roles.
//
//  K: the query of each head is a 31-bit fixed-point vector per 32-dim block (scale
//     S ~ max|q| / (127 2^24)) written as four signed digit bytes; the scores of 16 tokens
//     x 2 blocks are two v_mfma_i32_16x16x64_i8 (digits 0-1 and 2-3) whose rows are (head,
//     block, digit) and whose other operand is the unpacked codes (one byte each, in an
//     order fixed per code width that the query operand follows), so each lane scores one
//     head of one token.  The integer dot products are exact; the two 32-bit parts meet
//     in binary32, the code offset's share (o S sum(q_int)) is subtracted there (for KVarN
//     keys inside the integer sums), and the per-(token, block) scale applies afterwards.
//     Codes and scales go to registers, two or three steps in flight, through buffer loads
//     (non-temporal) that read rows past the end of a page as zero.
//  V: v_mfma_f32_4x4x4_16b_f16, one 4x4x4 block per (4-token group, 32-dim block): A =
//     the binary16 weights (2^15 p)(d 2^e) of the four heads (2^e a power of two uniform
//     over the wave, lowered when a larger block scale arrives, which keeps every weight
//     below 2^12 and far above the binary16 subnormals),
//     B = the centred codes 2^s (u - o) of one
//     dim per column as exact binary16 integers (v_perm interleaves the bytes of a token
//     pair; masking a code in place at bit offset s and or-ing 0x6400 gives 1024 + 2^s u,
//     one v_pk_add_f16 centres two codes; 2^-s is applied once at the end), K = the four
//     tokens.  The V rows
//     stream through a four-deep LDS ring filled by buffer loads straight to LDS, each
//     issued at the end of the step three before its use.
//  KVarN: keys are scored in the rotated domain with q'' = (H q / 128) * c_K of the page;
//     values accumulate in the rotated domain scaled by the page's c_V and are rotated
//     back once in the merge (x = H Yhat / 128, H the unnormalized Sylvester Hadamard
//     matrix).
//  kvarnN_1 (KVarN pages over affine blocks): keys add m * sum(q'') per block, taken from
//     each page's operand; the value minima are folded into the accumulator at every page
//     change, while it still carries that page's c_V.
//  Ring (BF16 tail) workgroups use the same pairing with binary32 arithmetic.
#pragma once

#include <float.h>
#include <type_traits>

#include "kvq_device.h"

namespace kvq {

namespace {

constexpr int kG = 4;
constexpr float kNeg = -1.0e30f;
constexpr float kQLim = 2130706432.0f;   // |q_int| bound 127 * 2^24: four balanced base-256 digits
constexpr int kP = 8;                    // (K wave, V wave) pairs per workgroup
constexpr float kPScale = 32768.0f;      // binary16 probabilities are stored as 2^15 p (p <= 1)
constexpr int kThreads = 128 * kP;       // one workgroup per CU

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));

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
constexpr int ROW_ROR1 = 0x121;     // row_ror:1
constexpr int ROW_ROR2 = 0x122;     // row_ror:2
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

// x with the value of lane l ^ 16 (or l ^ 32) combined in every lane, by v_permlane16_swap
// (v_permlane32_swap) with x as both operands: the two results then hold, in every lane, x
// of that lane and of its partner, with no LDS round trip (a shuffle is a ds_bpermute)
__device__ __forceinline__ float sum_x16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_x16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// reduction over lanes with equal (lane & 3)
__device__ __forceinline__ float wave_max16(float x)
{
    x = fmaxf(x, dpp<ROW_ROR4>(x));
    x = fmaxf(x, dpp<ROW_ROR8>(x));
    return max_x32(max_x16(x));
}
__device__ __forceinline__ float wave_sum16(float x)
{
    x += dpp<ROW_ROR4>(x);
    x += dpp<ROW_ROR8>(x);
    return sum_x32(sum_x16(x));
}
// reduction over lanes with equal (lane & 7)
__device__ __forceinline__ float wave_max8(float x)
{
    x = fmaxf(x, dpp<ROW_ROR8>(x));
    return max_x32(max_x16(x));
}
__device__ __forceinline__ float wave_sum8(float x)
{
    x += dpp<ROW_ROR8>(x);
    return sum_x32(sum_x16(x));
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

// Raw buffer resource over [p, p + bytes): loads at or past `bytes` return zero, so a
// step's loads need no clamping of rows past the end of a page.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
// The cache is read once per call: the key waves' loads are non-temporal (cache policy
// nt), measured 3 % faster than the default policy; the value rings' direct-to-LDS loads
// keep the default (nt on those measured no better, and slower together with nt keys).
constexpr int kNT = 2;                   // buffer-load cache policy: nt
__device__ __forceinline__ uint2 buf_load8(rsrc_t r, int off)
{
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNT));
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, int off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT));
}

// 16 bytes of global memory, non-temporal
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt16(const void* p)
{
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Buffer loads straight to LDS (lane l writes at lds + 16 l, or 4 l); like lds_load16, the
// waits are explicit.
__device__ __forceinline__ void lds_buf16(rsrc_t r, int voff, const void* lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds\n\ts_nop 0"
                 :: "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds))) : "memory", "m0");
}
__device__ __forceinline__ void lds_buf4(rsrc_t r, int voff, const void* lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds\n\ts_nop 0"
                 :: "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds))) : "memory", "m0");
}

__device__ __forceinline__ _Float16 lo_half(uint32_t w)
{
    return __builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ _Float16 hi_half(uint32_t w)
{
    return __builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Maximum over the 16 lanes of a DPP row, in every lane of the row: four v_max_f32 with a
// row rotation on the first operand (each preceded by the two wait states a DPP read of a
// just-written VGPR needs).  Finite inputs only.
__device__ __forceinline__ float row_max16(float x)
{
    asm volatile("s_nop 1\n\t"
                 "v_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
                 "s_nop 1\n\t"
                 "v_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
                 "s_nop 1\n\t"
                 "v_max_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
                 "s_nop 1\n\t"
                 "v_max_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf"
                 : "+v"(x));
    return x;
}

// One 32-token step of one value stream in LDS (NV-bit codes, rows of 16 NV bytes).  Code
// rows are stored even tokens first (rows 0..15 = tokens 0,2,..,30) then odd tokens (rows
// 16..31), so the value lanes read without bank conflicts; block-scale rows are in token
// order.
template <int NV>
struct alignas(16) Stage {
    uint8_t codes[32 * 16 * NV];
    uint8_t scales[32 * 16];
    uint16_t chan[128];
};
// LDS ring depth per value wave: four stages, three for 8-bit codes (LDS size)
template <int NV>
constexpr int ring_depth() { return NV == 8 ? 3 : 4; }

struct alignas(16) PBuf {
    union {
        float p[kG][32];     // [head][token of the step] probabilities of the step (ring)
        _Float16 ph[kG][32]; // the same in binary16 (quantized pages)
    };
    float alpha[4];          // accumulator rescale of the step (running max grew)
    float pad[4];
};

// Query operand of the score MFMA for one pair: 31-bit fixed-point query per (head, 32-dim
// block) as four balanced base-256 digits, q_int = d0 + 2^8 d1 + 2^16 d2 + 2^24 d3 with every
// d in [-128, 127], in the dim order in which the codes of each width unpack.
struct alignas(16) QMat {
    int8_t qa[4][kG][kD];    // [digit][head][permuted dim]
    float S[kG][4];          // [head][block] scale of q_int
    float qsum[kG][4];       // [head][block] S * sum(q_int)
    int sum[kG][4][2];       // [head][block] sums of the low (d0 + 2^8 d1) and high (d2 + 2^8 d3) parts
};

// The value accumulators a pair leaves at its end (wacc) live in the pair's own ring, which
// its value wave no longer reads once its loads have landed.
template <int NV>
struct alignas(16) WsLds {
    static constexpr int KS = ring_depth<NV>();
    union {
        float qs[kG][kD];    // the query of a ring workgroup
        QMat qm[kP];         // the score operand of each pair (quantized workgroups; KVarN
                             // rebuilds it two steps before each page, once the current
                             // page's operand is in registers)
    };
    Stage<NV> st[kP][KS];    // LDS rings of the value waves
    PBuf pb[kP][KS];         // [pair][step % KS]
    float wm[kP][kG], wl[kP][kG];
    __device__ float* wacc(int p) { return reinterpret_cast<float*>(&st[p][0]); }   // [kG][kD]
};
static_assert(sizeof(WsLds<6>) <= 160 * 1024 && sizeof(WsLds<8>) <= 160 * 1024, "LDS size");
static_assert(ring_depth<2>() * sizeof(Stage<2>) >= kG * kD * sizeof(float), "wacc fits a ring");

// x * (binary16 half of w), one v_fma_mix_f32 (no separate conversion).
__device__ __forceinline__ float mul_lo16(float x, uint32_t w)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(w));
    return r;
}
__device__ __forceinline__ float mul_hi16(float x, uint32_t w)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(w));
    return r;
}

// Maximum over the four lanes of a DPP quad (finite inputs).
__device__ __forceinline__ float quad_max(float x)
{
    asm volatile("s_nop 1\n\t"
                 "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
                 "s_nop 1\n\t"
                 "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
                 : "+v"(x));
    return x;
}

// ---- Key codes: the score operand of one lane --------------------------------------------
// Lane (token n, q) of the score MFMA supplies the 16 codes of half h = q & 1 of block
// 2 bp + (q >> 1): bits [16 N h, 16 N h + 16 N) of the block's N-bit little-endian stream.
// It loads the dword-aligned window that holds them (the data starts 16 h bits into it for
// N = 3) and unpacks them to one byte each; kpos<N> gives the byte position of element e
// (0..15) of the half, which the query operand follows.
template <int N>
constexpr int kwin_dwords() { return N == 2 ? 1 : N == 8 ? 4 : N >= 5 ? 3 : 2; }
// byte offset of lane half h's window within its block
template <int N>
__device__ __forceinline__ int kwin_off(int h) { return (2 * N * h) & ~3; }

template <int N>
__device__ __forceinline__ int kpos(int e)
{
    if constexpr (N == 2) return 4 * (e & 3) + (e >> 2);
    if constexpr (N == 3) {
        // element e -> position: dwords [e0 e8 e1 e9], [e3 e11 e4 e12], [e6 e14 e7 e15], [e2 e10 e5 e13]
        constexpr int t[16] = {0, 2, 12, 4, 6, 14, 8, 10, 1, 3, 13, 5, 7, 15, 9, 11};
        return t[e];
    }
    if constexpr (N == 4) {
        // dwords: low nibbles of bytes 0..3, high nibbles, then the same for bytes 4..7
        return (e < 8 ? 0 : 8) + ((e & 1) ? 4 : 0) + ((e & 7) >> 1);
    }
    if constexpr (N == 5) {
        // dwords [e0 e8 e2 e10], [e5 e13 e7 e15], [e1 e3 e4 e6], [e9 e11 e12 e14]
        constexpr int t[16] = {0, 8, 2, 9, 10, 4, 11, 6, 1, 12, 3, 13, 14, 5, 15, 7};
        return t[e];
    }
    if constexpr (N == 6) {
        // dwords [e0 e4 e3 e7], [e8 e12 e11 e15], [e1 e2 e5 e6], [e9 e10 e13 e14]
        constexpr int t[16] = {0, 8, 9, 2, 1, 10, 11, 3, 4, 12, 13, 6, 5, 14, 15, 7};
        return t[e];
    }
    return e;
}

// per-lane v_perm selectors and funnel shifts of the 3-bit unpack (they depend on h)
struct KSel { uint32_t a, b, c, y, y2; };
__device__ __forceinline__ KSel ksel3(int h)
{
    const uint32_t c = 2u * (uint32_t)h;          // byte offset of the data in the window
    auto two = [&](uint32_t b0, uint32_t b1) { return (c + b0) | ((c + b1) << 8) | ((c + b0) << 16) | ((c + b1) << 24); };
    return {two(0, 3), two(1, 4), two(2, 5), 6u + 8u * c, 15u + 8u * c};
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_shr16(uint32_t x, uint32_t s_lo, uint32_t s_hi)
{
    const u16x2 v = __builtin_bit_cast(u16x2, x);
    const u16x2 sh = {(unsigned short)s_lo, (unsigned short)s_hi};
    return __builtin_bit_cast(uint32_t, v >> sh);
}
__device__ __forceinline__ uint32_t pk_shl16(uint32_t x, uint32_t s_lo, uint32_t s_hi)
{
    const u16x2 v = __builtin_bit_cast(u16x2, x);
    const u16x2 sh = {(unsigned short)s_lo, (unsigned short)s_hi};
    return __builtin_bit_cast(uint32_t, v << sh);
}
__device__ __forceinline__ uint32_t bfe5(uint32_t x, uint32_t o) { return __builtin_amdgcn_ubfe(x, o, 5u); }

// The 16 codes of the lane's window as bytes (8-bit codes: u - 128 as a signed byte).
template <int N>
__device__ __forceinline__ i32x4 unpack_k(const uint32_t (&w)[kwin_dwords<N>()], const KSel& ks)
{
    if constexpr (N == 2) {
        const uint32_t m = 0x03030303u, x = w[0];
        return (i32x4){(int)(x & m), (int)((x >> 2) & m), (int)((x >> 4) & m), (int)((x >> 6) & m)};
    } else if constexpr (N == 3) {
        // elements at bit 3e: a 16-bit half of bytes (k, k + 3) shifted right by s holds the
        // two elements at offset s of those bytes in its two bytes when s <= 5; the four with
        // s = 6, 7 come from two funnel shifts of the window
        const uint32_t m = 0x07070707u;
        const uint32_t da = pk_shr16(__builtin_amdgcn_perm(w[1], w[0], ks.a), 0, 3) & m;
        const uint32_t db = pk_shr16(__builtin_amdgcn_perm(w[1], w[0], ks.b), 1, 4) & m;
        const uint32_t dc = pk_shr16(__builtin_amdgcn_perm(w[1], w[0], ks.c), 2, 5) & m;
        const uint32_t y = __builtin_amdgcn_alignbit(w[1], w[0], ks.y);
        const uint32_t y2 = __builtin_amdgcn_alignbit(w[1], w[0], ks.y2);
        const uint32_t dd = __builtin_amdgcn_perm(y2, y, 0x07040300u) & m;
        return (i32x4){(int)da, (int)db, (int)dc, (int)dd};
    } else if constexpr (N == 4) {
        const uint32_t m = 0x0F0F0F0Fu;
        return (i32x4){(int)(w[0] & m), (int)((w[0] >> 4) & m), (int)(w[1] & m), (int)((w[1] >> 4) & m)};
    } else if constexpr (N == 5) {
        // window data at bit 16 h: move it to bit 0 (x0..x2 = the 80 bits); codes at bit 5e.
        // Offsets s <= 3 of the pair bytes (k, k + 5) go through the half-word shift; the
        // eight codes that cross a byte are extracted one by one.
        const uint32_t sh = ks.y - 6u;                 // 16 h
        const uint32_t x0 = __builtin_amdgcn_alignbit(w[1], w[0], sh);
        const uint32_t x1 = __builtin_amdgcn_alignbit(w[2], w[1], sh);
        const uint32_t x2 = w[2] >> sh;
        const uint32_t m = 0x1F1F1F1Fu;
        const uint32_t d0 = pk_shr16(__builtin_amdgcn_perm(x1, x0, 0x06010500u), 0, 2) & m;
        const uint32_t z = __builtin_amdgcn_alignbit(x1, x0, 24);
        const uint32_t d1 = pk_shr16(__builtin_amdgcn_perm(x2, z, 0x05010400u), 1, 3) & m;
        const uint32_t e1 = bfe5(x0, 5), e3 = bfe5(x0, 15), e4 = bfe5(x0, 20);
        const uint32_t e6 = __builtin_amdgcn_alignbit(x1, x0, 30) & 31u;
        const uint32_t e9 = bfe5(x1, 13), e11 = bfe5(x1, 23), e14 = bfe5(x2, 6);
        const uint32_t e12 = __builtin_amdgcn_alignbit(x2, x1, 28) & 31u;
        const uint32_t d2 = (e1 | (e3 << 8)) | ((e4 | (e6 << 8)) << 16);
        const uint32_t d3 = (e9 | (e11 << 8)) | ((e12 | (e14 << 8)) << 16);
        return (i32x4){(int)d0, (int)d1, (int)d2, (int)d3};
    } else if constexpr (N == 6) {
        // codes at bit 6e, the window aligned; offsets 0 and 2 by the half-word shift of the
        // pair bytes, the codes that cross a byte from 16-bit windows shifted right (to bits
        // 0..5) or left (to bits 8..13) and merged with one bitfield insert
        const uint32_t x0 = w[0], x1 = w[1], x2 = w[2];
        const uint32_t m = 0x3F3F3F3Fu;
        const uint32_t da = pk_shr16(__builtin_amdgcn_perm(x1, x0, 0x05020300u), 0, 2) & m;
        const uint32_t db = pk_shr16(__builtin_amdgcn_perm(x2, x1, 0x07040502u), 0, 2) & m;
        const uint32_t w1 = pk_shr16(__builtin_amdgcn_perm(x1, x0, 0x04030100u), 6, 6);
        const uint32_t w2 = pk_shl16(__builtin_amdgcn_perm(x1, x0, 0x05040201u), 4, 4);
        const uint32_t dc = ((w1 & 0x00FF00FFu) | (w2 & 0xFF00FF00u)) & m;
        const uint32_t w3 = pk_shr16(__builtin_amdgcn_perm(x2, x1, 0x06050302u), 6, 6);
        const uint32_t w4 = pk_shl16(__builtin_amdgcn_perm(x2, x1, 0x07060403u), 4, 4);
        const uint32_t dd = ((w3 & 0x00FF00FFu) | (w4 & 0xFF00FF00u)) & m;
        return (i32x4){(int)da, (int)db, (int)dc, (int)dd};
    } else {
        const uint32_t f = 0x80808080u;
        return (i32x4){(int)(w[0] ^ f), (int)(w[1] ^ f), (int)(w[2] ^ f), (int)(w[3] ^ f)};
    }
}

// Fixed-point query operand (one page or the whole split).  Lane = head h (lane >> 4) x
// 8-dim group g8 (lane & 15); the four lanes of a quad hold one 32-dim block.  q: the lane's
// 8 query values; cw: the 8 key channel scales of the group (KVarN) or null.  The digits
// of element e of a half-block go to byte kpos<N>(e) of that half's 16 bytes.
//   q_int = rint(q * inv), inv = 127 * 2^24 / max|q| of the block; its balanced base-256
//   digits: d0 = the low byte of q_int, x1 = (q_int + 128) >> 8, d1 = the low byte of x1,
//   x2 = (x1 + 128) >> 8, and so on (arithmetic shifts), each digit in [-128, 127].  A
//   31-bit range keeps elements far below the block maximum (a key channel scale spread of
//   2^20 in a block, or a query outlier 1000x its block) with 8 or more significant bits.
template <int N>
__device__ __forceinline__ void build_qmat(QMat& Q, const float (&q)[8], const uint4* cw, int lane)
{
    const int h = lane >> 4, g8 = lane & 15, kb = g8 >> 2;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = q[e];
    if (cw) {
        const uint32_t cc[4] = {cw->x, cw->y, cw->z, cw->w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (e & 1) ? mul_hi16(v[e], cc[e >> 1]) : mul_lo16(v[e], cc[e >> 1]);
    }
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
    amax = fmaxf(fmaxf(amax, fabsf(v[3])), fabsf(v[4]));
    amax = fmaxf(fmaxf(amax, fabsf(v[5])), fabsf(v[6]));
    amax = quad_max(fmaxf(amax, fabsf(v[7])));
    // inv * amax <= 127 * 2^24 up to the rounding of the reciprocal: the bound is met with a
    // margin of 2^-7 (the top digit then stays within [-128, 127])
    const float inv = amax > 0.0f ? (kQLim * 0.9921875f) * __builtin_amdgcn_rcpf(amax) : 0.0f;
    // The four digits of q_int at once: y = q_int + 0x808080 carries every balanced digit's
    // +128 (bytes 0..2 of y are d0 + 128, d1 + 128, d2 + 128, and y >> 24 = d3), so
    // z = y ^ 0x808080 holds d0..d3 as its four two's-complement bytes, and the high part
    // d2 + 2^8 d3 = (y >> 16) - 128.  N = 4, 8: the lane's 8 elements fill 8 consecutive
    // bytes per digit ((even | odd) elements for N = 4, in order for N = 8): a 4 x 4 byte
    // transpose of four z's by v_perm per dword; other widths spread the positions over the
    // half-block, one byte store per digit.
    uint32_t z[8];
    uint32_t sx = 0u;                   // sum of q_int (mod 2^32)
    int shi = -8 * 128;                 // sum of the high parts
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int x = (int)__builtin_rintf(v[e] * inv);
        const int y = x + 0x808080;
        z[e] = (uint32_t)y ^ 0x808080u;
        sx += (uint32_t)x;
        shi += y >> 16;
        if constexpr (N != 4 && N != 8) {
            uint8_t* const bk = (uint8_t*)&Q.qa[0][h][16 * (g8 >> 1) + ((g8 & 1) ? kpos<N>(8 + e) : kpos<N>(e))];
#pragma unroll
            for (int k = 0; k < 4; ++k) bk[k * kG * kD] = (uint8_t)(z[e] >> (8 * k));
        }
    }
    // the sum of the low parts, d0 + 2^8 d1 = q_int - 2^16 (d2 + 2^8 d3), exact in 32 bits
    int slo = (int)(sx - ((uint32_t)shi << 16));
    if constexpr (N == 4 || N == 8) {
        // elements (a, b, c, d) -> dwords (digit 0 of a..d, digit 1, digit 2, digit 3)
        auto tr4 = [](uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t (&o)[4]) {
            const uint32_t t0 = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
            const uint32_t t1 = __builtin_amdgcn_perm(b, a, 0x07030602u);   // a2 b2 a3 b3
            const uint32_t u0 = __builtin_amdgcn_perm(d, c, 0x05010400u);   // c0 d0 c1 d1
            const uint32_t u1 = __builtin_amdgcn_perm(d, c, 0x07030602u);   // c2 d2 c3 d3
            o[0] = __builtin_amdgcn_perm(u0, t0, 0x05040100u);
            o[1] = __builtin_amdgcn_perm(u0, t0, 0x07060302u);
            o[2] = __builtin_amdgcn_perm(u1, t1, 0x05040100u);
            o[3] = __builtin_amdgcn_perm(u1, t1, 0x07060302u);
        };
        uint32_t w0[4], w1[4];
        if constexpr (N == 4) {
            tr4(z[0], z[2], z[4], z[6], w0);
            tr4(z[1], z[3], z[5], z[7], w1);
        } else {
            tr4(z[0], z[1], z[2], z[3], w0);
            tr4(z[4], z[5], z[6], z[7], w1);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) *(uint2*)&Q.qa[k][h][8 * g8] = make_uint2(w0[k], w1[k]);
    }
    slo += __builtin_amdgcn_mov_dpp(slo, QP_XOR1, 0xF, 0xF, false);
    slo += __builtin_amdgcn_mov_dpp(slo, QP_XOR2, 0xF, 0xF, false);
    shi += __builtin_amdgcn_mov_dpp(shi, QP_XOR1, 0xF, 0xF, false);
    shi += __builtin_amdgcn_mov_dpp(shi, QP_XOR2, 0xF, 0xF, false);
    if ((g8 & 3) == 0) {
        const float S = amax * (1.0f / (kQLim * 0.9921875f));
        Q.S[h][kb] = S;
        Q.qsum[h][kb] = S * fmaf((float)shi, 65536.0f, (float)slo);
        Q.sum[h][kb][0] = slo;
        Q.sum[h][kb][1] = shi;
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

// FK, FV: key and value formats (any quantized format, independently).
template <int FK, int FV>
__global__ __launch_bounds__(kThreads, 1) void k_decode_ws(DecodeArgs a)
{
    // KVARN_*: paged, rotated formats (kvarnN, kvarnN_1); AFF_*: affine blocks (qN_1, kvarnN_1)
    constexpr bool KVARN_K = kind_paged(fkind(FK)), KVARN_V = kind_paged(fkind(FV));
    constexpr bool AFF_K = kind_affine(fkind(FK)), AFF_V = kind_affine(fkind(FV));
    constexpr int NK = fbits(FK), NV = fbits(FV);
    constexpr int RK = 16 * NK, RV = 16 * NV;                       // code bytes per token row
    constexpr int SB_K = AFF_K ? 16 : 8, SB_V = AFF_V ? 16 : 8;   // scale bytes per token row
    constexpr int KS = ring_depth<NV>();                            // value ring depth
    constexpr int NI = (NV + 1) / 2;                                // code loads per value stage
    constexpr int kLoads = NI + 1 + (KVARN_V ? 1 : 0);              // V load instructions per stage
    static_assert(NK >= 2 && NK <= 8 && NK != 7 && NV >= 2 && NV <= 8 && NV != 7, "2- to 6- and 8-bit formats");

    __shared__ WsLds<NV> S;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bid = blockIdx.x;
    // Wave w runs on SIMD w % 4.  In each group of four waves two are K waves and two V
    // waves, on SIMDs (0, 1) and (2, 3) in even groups and the other way round in odd ones,
    // so every SIMD runs two waves of each role; pair 2g + b = the waves b and b + 2 of group g.
    const int wg4 = wave >> 2, w4 = wave & 3;
    const int pr = 2 * wg4 + (w4 & 1);
    const bool kwave = ((w4 >> 1) ^ (wg4 & 1)) == 0;
    const DecodeWork wk = decode_work(a, bid);
    const DecodeSeq& sq = a.seqs[wk.e];
    const int head = wk.head;
    const int sp = wk.sp;
    const bool quant = sp < sq.splits_q;
    const int upw = quant ? a.units_per_wg : a.units_per_wg_t;
    const int u_lo = (quant ? sp : sp - sq.splits_q) * upw;
    const int u_hi = min(u_lo + upw, quant ? sq.units_q : sq.units_t);
    const CacheGeom& g = a.g;
    const int nq = (int)sq.n_q;                      // token counts fit 31 bits
    const char* kst = sptr(g, sq.seq, a.layer, head, 0);
    const char* vst = sptr(g, sq.seq, a.layer, head, 1);

    // The query of the group, scaled to the log2 domain (KVarN pages: rotated, H q / 128),
    // into LDS.  Every role calls this once, after issuing its first loads, so that the
    // transform runs while they are in flight.
    auto load_query = [&]() {
        for (int i = tid; i < kG * kD; i += blockDim.x) {
            int hh = i / kD, d = i % kD;
            int64_t qi = ((int64_t)sq.in_idx * g.n_q_heads + head * kG + hh) * kD + d;
            float qv = a.q_dtype ? ((const float*)a.q)[qi] : bf16_to_f32(((const uint16_t*)a.q)[qi]);
            S.qs[hh][d] = qv * a.scale_log2;
        }
        __syncthreads();
        if (KVARN_K && quant) {
            lds_fwht4(S.qs);
            for (int i = tid; i < kG * kD; i += blockDim.x) S.qs[i / kD][i % kD] *= (1.0f / 128.0f);
            __syncthreads();
        }
    };

    // steps of each pair: the pair walks units u_lo + pr + kP i
    auto steps_of = [&](int p) -> int {
        const int uf = u_lo + p;
        if (uf >= u_hi) return 0;
        const int nu = (u_hi - uf + kP - 1) / kP;
        if (!quant) return nu;
        const int ul = uf + kP * (nu - 1);
        const int64_t len = min<int64_t>((int64_t)ul * kPage + kPage, sq.n_q) - (int64_t)ul * kPage;
        return 4 * (nu - 1) + (int)((len + 31) / 32);
    };
    const int J = steps_of(pr);
    int Jmax = 0;
    for (int p = 0; p < kP; ++p) Jmax = max(Jmax, steps_of(p));
    const int u_first = u_lo + pr;

    const int vg = lane >> 3, vp = lane & 7;          // V layout: pair slot (of 8), 16-dim part
    const int vb = vp >> 1;

    // end of a role: the K wave leaves (m, l) per head, the V wave its slot-summed accumulator
    // end of a ring role: the K wave leaves (m, l) per head, the V wave its slot-summed
    // accumulator (lane h < 4 of the K wave holds head h)
    auto finish_k = [&](float mv, float lsum) {
        const float t = wave_sum8(vp < kG ? lsum : 0.0f);
        if (lane < kG) {
            S.wl[pr][lane] = t;
            S.wm[pr][lane] = mv;
        }
    };
    auto finish_v = [&](float (&acc)[kG][16]) {
#pragma unroll
        for (int h = 0; h < kG; ++h)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const float y = wave_sum8(acc[h][jj]);
                if (vg == 0) S.wacc(pr)[h * kD + 16 * vp + jj] = y;
            }
    };
    if (quant && kwave) {
        // ============================ K wave (MFMA scores) ============================
        // One v_mfma_i32_16x16x64_i8 per (16-token tile, block pair): rows = (head, block of
        // the pair, byte of q_int), columns = tokens, K = the 64 dims of the two blocks (a row
        // is zero over the other block's dims).  Lane (n = lane & 15, q = lane >> 4) supplies
        // the codes of token n, dims 16q..16q+15 of the pair, and receives rows 4q..4q+3:
        // head q, both blocks of the pair, both bytes.  So a lane scores one head of one token
        // per tile on its own, and the running maximum of a head is a 16-lane row reduction.
        // The MFMA accumulator starts at -o sum(q_int) of the block for symmetric codes with
        // offset o = 2^(N-1), which takes the offset out of the integer sum (8-bit codes enter
        // as u - 128 already; affine 8-bit keys add 128 sum(q_int) back).
        constexpr int KWD = kwin_dwords<NK>();
        constexpr int OFF_K = NK == 8 ? (AFF_K ? -128 : 0) : (AFF_K ? 0 : 1 << (NK - 1));
        const int n16 = lane & 15, q4 = lane >> 4;
        const KSel ks = ksel3(q4 & 1);
        const char* kcodes = kst + g.k.codes;
        const char* kscales = kst + g.k.scales;
        const char* kchan = kst + g.k.cscale;
        QMat& Qb = S.qm[pr];
        // A[bp] / A2[bp]: digits (0, 1) / (2, 3) of the rows.  The code offset o: for block
        // formats a binary32 term -o S sum(q_int) per block (Qo); for KVarN keys, whose query
        // operand carries the channel scales (elements up to 10^4 or more beside small
        // centred codes, where that term would cancel), exactly in the integer sums: the low
        // part's share in the accumulator (Ci), the high part's subtracted before the parts
        // meet (Oh).  The affine minimum enters as S sum(q_int) (Qs) times the block's m.
        i32x4 A[2], A2[2];
        float Sc[4], Qs[4], Qo[4];
        i32x4 Ci[KVARN_K ? 2 : 1];
        int Oh[KVARN_K ? 2 : 1][2];
        auto load_a = [&](const QMat& Q) {
            const int m = n16, dig = m & 1, sel = (m >> 1) & 1, h = m >> 2;
#pragma unroll
            for (int bp = 0; bp < 2; ++bp) {
                const i32x4 z = {0, 0, 0, 0};
                const int o = 32 * (2 * bp + sel) + 16 * (q4 & 1);
                A[bp] = sel == (q4 >> 1) ? *(const i32x4*)&Q.qa[dig][h][o] : z;
                A2[bp] = sel == (q4 >> 1) ? *(const i32x4*)&Q.qa[2 + dig][h][o] : z;
                if constexpr (KVARN_K) {
                    Ci[bp] = (i32x4){-OFF_K * Q.sum[q4][2 * bp][0], 0, -OFF_K * Q.sum[q4][2 * bp + 1][0], 0};
                    Oh[bp][0] = OFF_K * Q.sum[q4][2 * bp][1];
                    Oh[bp][1] = OFF_K * Q.sum[q4][2 * bp + 1][1];
                }
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                Sc[b] = Q.S[q4][b];
                // affine keys: the sum of the rounded query, S * sum(q_int), so that the score
                // is the rounded query against the dequantized key, d u + m, exactly; its
                // error is then sum((q - q_hat) k), small where a block holds one outlier
                // channel (the other keys are near 0, while d u - 8 d or d u are not)
                Qs[b] = AFF_K ? Q.qsum[q4][b] : 0.0f;
                Qo[b] = KVARN_K ? 0.0f : (float)(-OFF_K) * Q.qsum[q4][b];
            }
        };
        // Codes and scales of one step, straight to registers through buffer loads whose
        // resource covers the step's valid tokens: rows past the end of the page read as zero
        // (their scores are masked).  Stages past the last step repeat it.
        // ch (KVarN): the key channel scales of the page after the step's page, loaded with the
        // step's rows so that the waits the compiler places for them stay exact
        struct KLoad { uint32_t c[2][2][KWD]; uint4 s[2]; uint4 ch; };
        const int cofs = n16 * RK + 4 * NK * (q4 >> 1) + kwin_off<NK>(q4 & 1), sofs = n16 * SB_K;
        auto chan_load = [&](int i) -> uint4 {      // key channel scales of the pair's i-th page
            const int nu = (u_hi - u_first + kP - 1) / kP;
            const int u = u_first + kP * min(i, nu - 1);
            return *(const uint4*)(kchan + (int64_t)u * 256 + 16 * (lane & 15));
        };
        auto kload = [&](int j, KLoad& L) {
            const int jj = j < J ? j : J - 1;
            const int u = u_first + kP * (jj >> 2);
            const int tb = u * kPage + 32 * (jj & 3);
            const int nv = min(32, min(u * kPage + kPage, nq) - tb);
            const rsrc_t rc = make_rsrc(kcodes + (int64_t)tb * RK, nv * RK);
            const rsrc_t rs = make_rsrc(kscales + (int64_t)tb * SB_K, nv * SB_K);
#pragma unroll
            for (int T = 0; T < 2; ++T) {
#pragma unroll
                for (int bp = 0; bp < 2; ++bp) {
                    const int o = cofs + 16 * RK * T + 8 * NK * bp;
                    if constexpr (KWD == 1) {
                        L.c[T][bp][0] = __builtin_amdgcn_raw_buffer_load_b32(rc, o, 0, kNT);
                    } else if constexpr (KWD == 2) {
                        const uint2 x = buf_load8(rc, o);
                        L.c[T][bp][0] = x.x; L.c[T][bp][1] = x.y;
                    } else if constexpr (KWD == 3) {
                        const auto x = __builtin_amdgcn_raw_buffer_load_b96(rc, o, 0, kNT);
                        L.c[T][bp][0] = x[0]; L.c[T][bp][1] = x[1]; L.c[T][bp][2] = x[2];
                    } else {
                        const uint4 x = buf_load16(rc, o);
                        L.c[T][bp][0] = x.x; L.c[T][bp][1] = x.y; L.c[T][bp][2] = x.z; L.c[T][bp][3] = x.w;
                    }
                }
                if (AFF_K) {
                    L.s[T] = buf_load16(rs, sofs + 16 * SB_K * T);
                } else {
                    const uint2 w = buf_load8(rs, sofs + 16 * SB_K * T);
                    L.s[T] = make_uint4(w.x, w.y, 0u, 0u);
                }
            }
            if (KVARN_K) L.ch = chan_load((jj >> 2) + 1);
        };
        float mh = kNeg;                           // running max of head q4
        float ls = 0.0f;                           // sum of p over the lane's tokens
        uint4 cfirst = make_uint4(0u, 0u, 0u, 0u);
        // three register stages, loads issued two steps ahead of their use
        // KR register stages (two where three would not fit in the registers: wide KVarN keys)
        constexpr int KR = KVARN_K ? 2 : 3;
        KLoad X, Y, Z;
        if (J > 0) {
            if (KVARN_K) cfirst = chan_load(0);        // first, so that its wait is exact
            kload(0, X);
            kload(1, Y);
            if (KR == 3) kload(2, Z);
        }
        // the lane's 8 query values (head lane >> 4, dims 8 (lane & 15) ..), log2 domain;
        // KVarN: rotated, H q / 128 (spans 1, 2, 4 in the lane, 8 .. 64 across lanes)
        float qv[8];
        {
            const int64_t qi = ((int64_t)sq.in_idx * g.n_q_heads + head * kG + (lane >> 4)) * kD + 8 * n16;
            if (a.q_dtype) {
                const float4 x0 = *(const float4*)((const float*)a.q + qi);
                const float4 x1 = *(const float4*)((const float*)a.q + qi + 4);
                qv[0] = x0.x; qv[1] = x0.y; qv[2] = x0.z; qv[3] = x0.w;
                qv[4] = x1.x; qv[5] = x1.y; qv[6] = x1.z; qv[7] = x1.w;
            } else {
                const uint4 w = *(const uint4*)((const uint16_t*)a.q + qi);
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qv[2 * i] = bf16_to_f32(ww[i] & 0xFFFFu);
                    qv[2 * i + 1] = bf16_to_f32(ww[i] >> 16);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[e] *= a.scale_log2;
            if (KVARN_K) {
#pragma unroll
                for (int sp = 1; sp < 8; sp <<= 1)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if ((e & sp) == 0) {
                            const float x = qv[e], y = qv[e + sp];
                            qv[e] = x + y;
                            qv[e + sp] = x - y;
                        }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const bool up = (lane >> k) & 1;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float y = __shfl_xor(qv[e], 1 << k);
                        qv[e] = up ? y - qv[e] : qv[e] + y;
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) qv[e] *= (1.0f / 128.0f);
            }
        }
        if (!KVARN_K) {
            build_qmat<NK>(Qb, qv, nullptr, lane);
            wave_sync_lds();
            load_a(Qb);
        } else if (J > 0) {
            // first page now; each later page's operand is built two steps before it starts,
            // over the current page's, which is in registers by then (a wave's LDS accesses
            // complete in order)
            build_qmat<NK>(Qb, qv, &cfirst, lane);
            wave_sync_lds();
            load_a(Qb);
        }
        // slot: the probability buffer of step j, j % KS
        auto kstep = [&](int j, const KLoad& L, int slot) __attribute__((always_inline)) {
            const int u = u_first + kP * (j >> 2);
            const int t_page = u * kPage;
            const int t_end = min(t_page + kPage, nq);
            if (KVARN_K && (j & 3) == 0 && j > 0) {
                wave_sync_lds();
                load_a(Qb);
            }
            if (KVARN_K && (j & 3) == 2) {
                // the next page's operand into the other buffer (read at that page's start)
                build_qmat<NK>(Qb, qv, &L.ch, lane);
            }
            float sc[2];
#pragma unroll
            for (int T = 0; T < 2; ++T) {
                float acc = 0.0f;
#pragma unroll
                for (int bp = 0; bp < 2; ++bp) {
                    const i32x4 Bm = unpack_k<NK>(L.c[T][bp], ks);
                    const i32x4 z4 = {0, 0, 0, 0};
                    // integer dot of each block, sum(q_int (u - o)): the low (digits 0, 1) and
                    // high (digits 2, 3) parts are exact in 32 bits and meet in binary32
                    float t0, t1;
                    if constexpr (KVARN_K) {
                        const i32x4 C = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[bp], Bm, Ci[bp], 0, 0, 0);
                        const i32x4 C2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A2[bp], Bm, z4, 0, 0, 0);
                        t0 = fmaf((float)((C2.y << 8) + C2.x - Oh[bp][0]), 65536.0f, (float)((C.y << 8) + C.x)) * Sc[2 * bp];
                        t1 = fmaf((float)((C2.w << 8) + C2.z - Oh[bp][1]), 65536.0f, (float)((C.w << 8) + C.z)) * Sc[2 * bp + 1];
                    } else {
                        const i32x4 C = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[bp], Bm, z4, 0, 0, 0);
                        const i32x4 C2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A2[bp], Bm, z4, 0, 0, 0);
                        t0 = fmaf(fmaf((float)((C2.y << 8) + C2.x), 65536.0f, (float)((C.y << 8) + C.x)), Sc[2 * bp], Qo[2 * bp]);
                        t1 = fmaf(fmaf((float)((C2.w << 8) + C2.z), 65536.0f, (float)((C.w << 8) + C.z)), Sc[2 * bp + 1], Qo[2 * bp + 1]);
                    }
                    // block scales as binary16 operands of v_fma_mix (no conversion)
                    uint32_t w0, w1;
                    if (AFF_K) {
                        w0 = bp ? L.s[T].z : L.s[T].x;
                        w1 = bp ? L.s[T].w : L.s[T].y;
                        acc = fmaf(t0, (float)lo_half(w0), acc);
                        acc = fmaf(t1, (float)lo_half(w1), acc);
                        acc = fmaf(Qs[2 * bp], (float)hi_half(w0), acc);
                        acc = fmaf(Qs[2 * bp + 1], (float)hi_half(w1), acc);
                    } else {
                        w0 = bp ? L.s[T].y : L.s[T].x;
                        acc = fmaf(t0, (float)lo_half(w0), acc);
                        acc = fmaf(t1, (float)hi_half(w0), acc);
                    }
                }
                sc[T] = acc;
            }
            if (t_end - (t_page + 32 * (j & 3)) < 32) {
                // the page ends inside this step: mask the rows past its end
#pragma unroll
                for (int T = 0; T < 2; ++T)
                    if (t_page + 32 * (j & 3) + 16 * T + n16 >= t_end) sc[T] = kNeg;
            }
            // running max of head q4 (a 16-lane row): once the first steps have set it, a new
            // maximum is rare, so the row reduction and the rescale factor are only computed
            // when some lane's score exceeds it (the result is the same either way)
            float al = 1.0f;
            if (__builtin_amdgcn_ballot_w64(fmaxf(sc[0], sc[1]) > mh)) {
                const float nm = fmaxf(mh, row_max16(fmaxf(sc[0], sc[1])));
                al = __builtin_amdgcn_exp2f(mh - nm);                // exactly 1 if unchanged
                mh = nm;
            }
            const float p0 = __builtin_amdgcn_exp2f(sc[0] - mh);
            const float p1 = __builtin_amdgcn_exp2f(sc[1] - mh);
            ls = fmaf(ls, al, p0 + p1);
            PBuf& P = S.pb[pr][slot];
            P.ph[q4][n16] = (_Float16)(p0 * kPScale);
            P.ph[q4][16 + n16] = (_Float16)(p1 * kPScale);
            if (n16 == 0) P.alpha[q4] = al;
            __syncthreads();
        };
        int j = 0;
        if constexpr (KR == 3) {
#pragma unroll 1
            for (; j + 2 < J; j += 3) {
                kstep(j, X, KS == 3 ? 0 : j & 3);
                kload(j + 3, X);
                kstep(j + 1, Y, KS == 3 ? 1 : (j + 1) & 3);
                kload(j + 4, Y);
                kstep(j + 2, Z, KS == 3 ? 2 : (j + 2) & 3);
                kload(j + 5, Z);
            }
            if (j < J) { kstep(j, X, KS == 3 ? 0 : j & 3); ++j; }
            if (j < J) { kstep(j, Y, KS == 3 ? 1 : j & 3); ++j; }
        } else {
#pragma unroll 1
            for (; j + 1 < J; j += 2) {
                kstep(j, X, j % KS);
                kload(j + 2, X);
                kstep(j + 1, Y, (j + 1) % KS);
                kload(j + 3, Y);
            }
            if (j < J) { kstep(j, X, j % KS); ++j; }
        }
#pragma unroll 1
        for (; j <= Jmax; ++j) __syncthreads();
        // normalizer of head q4 over its row
        float l = ls;
        l += dpp<ROW_ROR8>(l);
        l += dpp<ROW_ROR4>(l);
        l += dpp<ROW_ROR2>(l);
        l += dpp<ROW_ROR1>(l);
        if (n16 == 0) {
            S.wl[pr][q4] = l;
            S.wm[pr][q4] = mh;
        }
    } else if (quant) {
        // ================================ V wave ================================
        const char* cbase = vst + g.v.codes;
        const char* sbase = vst + g.v.scales;
        const char* chbase = vst + g.v.cscale;
        Stage<NV>* ring = S.st[pr];
        // stage j -> ring slot j % KS; the number of load instructions per stage is fixed
        // (stages past the end repeat the last), so one vmcnt value covers a stage.  Buffer
        // resources over the step's valid rows: rows past the end of the page read as zero
        // (the ring is zeroed first, so no slot ever holds non-finite bytes either way; the
        // weights of those rows are zero).  Codes: the stage's 32 NV chunks of 16 bytes, lane
        // l of load i taking chunk c = 64 i + l (LDS bytes 16 c, so LDS row c / NV); LDS row r
        // holds token 2 r (r < 16) or 2 (r - 16) + 1.
        int voff[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = 64 * i + lane, row = c / NV;
            voff[i] = (row < 16 ? 2 * row : 2 * (row - 16) + 1) * RV + 16 * (c % NV);
        }
        auto issue = [&](int j, int slot) {
            const int jj = j < J ? j : J - 1;
            const int u = u_first + kP * (jj >> 2);
            const int tb = u * kPage + 32 * (jj & 3);
            const int nv = min(32, min(u * kPage + kPage, nq) - tb);
            Stage<NV>& B = ring[slot];
            const rsrc_t rc = make_rsrc(cbase + (int64_t)tb * RV, nv * RV);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const bool full = 64 * (i + 1) <= 32 * NV;       // else lanes < 32 (odd NV)
                if (full || lane < 32 * NV - 64 * i) lds_buf16(rc, voff[i], B.codes + 1024 * i);
            }
            const rsrc_t rs = make_rsrc(sbase + (int64_t)tb * SB_V, nv * SB_V);
            if (AFF_V) {
                if (lane < 32) lds_buf16(rs, 16 * lane, B.scales);
            } else {
                lds_buf4(rs, 4 * lane, B.scales);
            }
            if (KVARN_V) {
                if (lane < 16) lds_buf16(make_rsrc(chbase + (int64_t)u * 256, 256), 16 * lane, B.chan);
            }
        };
        {
            // zero the ring once
            uint4* z = (uint4*)ring;
            for (int i = lane; i < (int)(KS * sizeof(Stage<NV>) / 16); i += 64) z[i] = make_uint4(0u, 0u, 0u, 0u);
            wave_sync_lds();
        }
        if (J > 0) {
#pragma unroll
            for (int i = 0; i < KS - 1; ++i) issue(i, i);
        }
        // Lane = (token group tg = lane >> 4, block vblk = (lane >> 2) & 3, slice vj = lane & 3)
        // owns dims 32 vblk + 8 vj .. + 7 (its "run": N bytes of a code row).  In half `hf` of a
        // step the group takes the token pairs s0 = 8 hf + tg and s1 = s0 + 4 (tokens 2 s0,
        // 2 s0 + 1, 2 s1, 2 s1 + 1).  MFMA block (tg, vblk) = lanes 4 (lane >> 2) .. + 3: A row
        // i = the binary16 weights p d of head i for the four tokens, B column i = the centred
        // codes of dim 32 vblk + 8 i + r (r = 0..7, one MFMA each), K = the four tokens; D
        // column i accumulates the four heads of that dim.  Centring before the sum matters at
        // long context: with spread attention the output is far smaller than sum(w u) or
        // o sum(w), and the fp32 rounding of either would be amplified.
        // Code r of a run sits at bit N r: byte (N r) >> 3, offset s = (N r) & 7.  v_perm puts
        // that byte (and the next, where a 3-bit code crosses into it) of both tokens of a pair
        // in the two 16-bit halves; masking the code in place and or-ing 0x6400 gives the
        // binary16 value 1024 + 2^s u, exact since 2^s u < 1024; one packed add makes it
        // 2^s (u - o), o = 2^(N-1), also exact.  The factor 2^s of each dim is removed at the end.
        const int tg = lane >> 4, vblk = (lane >> 2) & 3, vj = lane & 3;
        const int lrun = 4 * NV * vblk + NV * vj;          // byte offset of the run in a row
        struct VRun { uint32_t x[NV == 8 ? 2 : (NV == 5 || NV == 6) ? 3 : 1]; };
        auto vrun = [&](const uint8_t* cb, int row) -> VRun {
            VRun R;
            const int o = row * RV + lrun;
            if constexpr (NV == 8) {
                const uint2 w = *(const uint2*)(cb + o);
                R.x[0] = w.x; R.x[1] = w.y;
            } else if constexpr (NV == 4) {
                R.x[0] = *(const uint32_t*)(cb + o);
            } else if constexpr (NV == 2) {
                R.x[0] = *(const uint32_t*)(cb + (o & ~3)) >> (8 * (lrun & 3));
            } else if constexpr (NV == 5 || NV == 6) {
                // 40 or 48 bits: R0 = bytes 0..3, R1 = bytes 4..7, Rm = bytes 3..6 of the run
                const uint32_t* w = (const uint32_t*)(cb + (o & ~3));
                const uint32_t d0 = w[0], d1 = w[1], sh = 8 * (lrun & 3);
                R.x[0] = __builtin_amdgcn_alignbit(d1, d0, sh);
                R.x[1] = d1 >> sh;
                R.x[2] = __builtin_amdgcn_alignbit(R.x[1], R.x[0], 24);
            } else {
                const uint32_t* w = (const uint32_t*)(cb + (o & ~3));
                R.x[0] = __builtin_amdgcn_alignbit(w[1], w[0], 8 * (lrun & 3));
            }
            return R;
        };
        f32x4 D[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) D[r] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        float ms = 0.0f, msd = 0.0f;  // sums of p m and p d of head vj over the lane's tokens (affine)
        float cvr[8];                 // c_V of the lane's dims on the current page (KVarN)
#pragma unroll
        for (int r = 0; r < 8; ++r) cvr[r] = 1.0f;
        // Value-weight exponent of the wave: the weights enter the MFMA as binary16
        // (2^15 p) * (d 2^ve), with d 2^ve < 2^-3 for every block scale the wave has seen, so
        // a weight stays below 2^12 and far above the binary16 subnormals whatever the
        // magnitude of the values.  ve starts at 15 and only decreases: when a step brings a
        // larger scale, ve drops so that the largest scale sits in [2^-5, 2^-4) and the
        // accumulator (binary32) is rescaled by the exact power of two.  ve is uniform over
        // the wave (scalar registers).
        int ve = 15;
        // 0x64006400 kept in a register so that the mask-and-or is one v_and_or_b32
        uint32_t k6400 = 0x64006400u;
        asm volatile("" : "+v"(k6400));
        // binary16 pair of code r of tokens a (low half) and b (high half), centred and scaled
        // by 2^s', s' = min(s, 10 - N) (a window whose code sits higher is shifted down first)
        auto vcode = [&](const VRun& ra, const VRun& rb, int r) __attribute__((always_inline)) -> half2_t {
            constexpr int kM = (1 << NV) - 1;
            const int bit = NV * r, k = bit >> 3, s = bit & 7;
            const int s2 = s < 10 - NV ? s : 10 - NV;
            const _Float16 c = (_Float16)(-(1024.0f + (float)((1 << (NV - 1)) << s2)));
            const half2_t cc = {c, c};
            uint32_t w;
            if constexpr (NV == 5 || NV == 6) {
                // window (k, k + 1) of the run: bytes of R0 (k <= 2), Rm (k = 3) or R1 (k >= 4)
                const int src = k <= 2 ? 0 : k == 3 ? 2 : 1;
                const uint32_t kk = (uint32_t)(k <= 2 ? k : k == 3 ? 0 : k - 4);
                const uint32_t sel = kk | ((kk + 1) << 8) | ((4 + kk) << 16) | ((5 + kk) << 24);
                uint32_t x = __builtin_amdgcn_perm(rb.x[src], ra.x[src], sel);
                if (s > s2) x >>= (s - s2);
                w = (x & ((uint32_t)(kM << s2) * 0x00010001u)) | k6400;
            } else if constexpr (NV == 8) {
                w = __builtin_amdgcn_perm(rb.x[k >> 2], ra.x[k >> 2],
                                          (uint32_t)(k & 3) | 0x0C000C00u | ((uint32_t)(4 + (k & 3)) << 16)) | k6400;
            } else {
                const bool cross = s + NV > 8;            // 3-bit codes at offsets 6 and 7
                const uint32_t sel = (uint32_t)k | ((uint32_t)(4 + k) << 16) |
                                     (cross ? (((uint32_t)(k + 1) << 8) | ((uint32_t)(5 + k) << 24)) : 0x0C000C00u);
                const uint32_t m = (uint32_t)(kM << s) * 0x00010001u;
                w = (__builtin_amdgcn_perm(rb.x[0], ra.x[0], sel) & m) | k6400;
            }
            return __builtin_bit_cast(half2_t, w) + cc;
        };
        auto quad_bcast = [&](float x, int h) -> float {     // lane h of the lane's quad
            return h == 0 ? dpp<0x00>(x) : h == 1 ? dpp<0x55>(x) : h == 2 ? dpp<0xAA>(x) : dpp<0xFF>(x);
        };
        // Stage j + KS - 1 is issued at the end of step j, once the step's LDS reads are done:
        // a global-to-LDS load in flight holds lgkmcnt for a while after issue, and every LDS
        // wait of the step would pay for it.  The V wave publishes nothing through LDS, so its
        // barrier needs no lgkmcnt wait (bare s_barrier; the clobber keeps the compiler from
        // moving LDS accesses across it).
        auto vstep = [&](int j, int slot) __attribute__((always_inline)) {
            const bool page_start = (j & 3) == 0;
            wait_vmcnt<(KS - 2) * kLoads>();
            asm volatile("" ::: "memory");
            const Stage<NV>& B = ring[slot];
            const PBuf& P = S.pb[pr][slot];
            // the step's block scales (two token pairs per half), gathered by 16-bit LDS loads
            const _Float16* sc16 = (const _Float16*)B.scales;
            constexpr int SW = SB_V / 2;                       // binary16 words per scale row
            const int so = (AFF_V ? 2 : 1) * vblk;
            auto dpair = [&](int hf, int i) __attribute__((always_inline)) -> half2_t {
                const int sx = 8 * hf + tg + 4 * i;
                return (half2_t){sc16[SW * (2 * sx) + so], sc16[SW * (2 * sx + 1) + so]};
            };
            // the scales of the range check below are read together with the rescale factor,
            // so that one LDS wait covers both
            const half2_t dq0 = dpair(0, 0), dq1 = dpair(0, 1), dq2 = dpair(1, 0), dq3 = dpair(1, 1);
            // KVarN: this page's value channel scales of the lane's dims, read with them
            const uint4 cpg = KVARN_V && page_start ? *(const uint4*)(B.chan + 32 * vblk + 8 * vj)
                                                    : make_uint4(0u, 0u, 0u, 0u);
            // the MFMA operands of both halves of the step (codes of the lane's runs, binary16
            // 2^15 p): for symmetric block values (qN_0) of up to 4 bits they are read here
            // too, so the whole step waits on one batch of LDS reads (q4_0, q2_0: +5-6 %);
            // other formats read them per half (measured 0.7 % slower early for kvarn4, whose
            // page-start rescale keeps more registers live)
            constexpr bool kOpsEarly = !AFF_V && !KVARN_V && NV <= 4;
            struct VOps { VRun x[4]; half2_t p01, p23; };
            auto read_ops = [&](int hf) __attribute__((always_inline)) -> VOps {
                const int s0 = 8 * hf + tg, s1 = s0 + 4;
                VOps o;
                o.x[0] = vrun(B.codes, s0);
                o.x[1] = vrun(B.codes, 16 + s0);
                o.x[2] = vrun(B.codes, s1);
                o.x[3] = vrun(B.codes, 16 + s1);
                o.p01 = *(const half2_t*)&P.ph[vj][2 * s0];
                o.p23 = *(const half2_t*)&P.ph[vj][2 * s1];
                return o;
            };
            VOps early[2];
            if constexpr (kOpsEarly) {
                early[0] = read_ops(0);
                early[1] = read_ops(1);
            }
            const f32x4 al = *(const f32x4*)P.alpha;
            if (al.x != 1.0f || al.y != 1.0f || al.z != 1.0f || al.w != 1.0f) {
#pragma unroll
                for (int r = 0; r < 8; ++r) D[r] *= al;
                ms *= al[vj];
                msd *= al[vj];
            }
            if (KVARN_V && AFF_V && page_start) {
                // kvarnN_1 values: the minima summed so far carry the previous page's channel
                // scales, so they join the accumulator (at its 2^s' code scale) before it moves
                // to this page's; the lane's partial sums, like its accumulator's
                // (the sums carry the 2^15 of the probabilities, the accumulator also 2^ve)
                const float mo = fmaf((float)(1 << (NV - 1)), msd, ms) * __builtin_ldexpf(1.0f, ve);
                const f32x4 m4 = {quad_bcast(mo, 0), quad_bcast(mo, 1), quad_bcast(mo, 2), quad_bcast(mo, 3)};
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int s = (NV * r) & 7;
                    D[r] += m4 * (float)(1 << (s < 10 - NV ? s : 10 - NV));
                }
                ms = 0.0f;
                msd = 0.0f;
            }
            if (KVARN_V && page_start) {
                // this page's value channel scales: move the accumulator to them (it is zero
                // before the first page, so the first move is inert)
                const uint32_t cw[4] = {cpg.x, cpg.y, cpg.z, cpg.w};
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const float cn = fp16_to_f32((cw[r >> 1] >> (16 * (r & 1))) & 0xFFFFu);
                    D[r] *= cvr[r] * __builtin_amdgcn_rcpf(cn);
                    cvr[r] = cn;
                }
            }
            {
                // a scale of the step at or above 2^(-3 - ve): lower ve for the whole wave
                const u16x2 m = {0x7FFF, 0x7FFF};
                u16x2 r = __builtin_bit_cast(u16x2, dq0) & m;
                r = __builtin_elementwise_max(r, __builtin_bit_cast(u16x2, dq1) & m);
                r = __builtin_elementwise_max(r, __builtin_bit_cast(u16x2, dq2) & m);
                r = __builtin_elementwise_max(r, __builtin_bit_cast(u16x2, dq3) & m);
                const uint32_t dm = r.x > r.y ? r.x : r.y;  // binary16 bits of the largest |d|
                const uint32_t lim = (uint32_t)max(0, 12 - ve) << 10;     // 2^(-3 - ve)
                if (__builtin_amdgcn_ballot_w64(dm >= lim)) {
                    // the wave's largest scale in [2^e, 2^(e+1)) (binary16 subnormals: e = -14
                    // bounds them); ve puts it in [2^-5, 2^-4)
                    uint32_t wm = dm;
#pragma unroll
                    for (int o = 32; o >= 1; o >>= 1) wm = max(wm, (uint32_t)__shfl_xor((int)wm, o));
                    const int ef = (int)(__builtin_amdgcn_readfirstlane(wm) >> 10);
                    const int nve = max(-24, -5 - ((ef == 0 ? 1 : ef) - 15));
                    const float f = __builtin_ldexpf(1.0f, nve - ve);
#pragma unroll
                    for (int r2 = 0; r2 < 8; ++r2) D[r2] *= f;
                    ve = nve;
                }
            }
            // affine values reload the scales below (registers); the others keep the four read
            // above, and their operand reads below may move up past the checks
            if constexpr (AFF_V) asm volatile("" ::: "memory");
            const uint32_t vh = ve >= -14 ? (uint32_t)(ve + 15) << 10 : 1u << (ve + 24);
            const half2_t vsc = __builtin_bit_cast(half2_t, vh | (vh << 16));   // {2^ve, 2^ve}
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int s0 = 8 * hf + tg, s1 = s0 + 4;
                const VOps ops = kOpsEarly ? early[hf] : read_ops(hf);
                const VRun &x0 = ops.x[0], &x1 = ops.x[1], &x2 = ops.x[2], &x3 = ops.x[3];
                // A: binary16 2^15 p (written by the K wave) times the scaled binary16 block
                // scales, two tokens per packed multiply
                const half2_t p01 = ops.p01, p23 = ops.p23;
                uint32_t a01, a23;
                if constexpr (AFF_V) {
                    a01 = __builtin_bit_cast(uint32_t, p01 * (dpair(hf, 0) * vsc));
                    a23 = __builtin_bit_cast(uint32_t, p23 * (dpair(hf, 1) * vsc));
                } else {
                    a01 = __builtin_bit_cast(uint32_t, p01 * ((hf ? dq2 : dq0) * vsc));
                    a23 = __builtin_bit_cast(uint32_t, p23 * ((hf ? dq3 : dq1) * vsc));
                }
                if (AFF_V) {
                    const half2_t d01 = dpair(hf, 0), d23 = dpair(hf, 1);
                    const half2_t m01 = {sc16[SW * (2 * s0) + so + 1], sc16[SW * (2 * s0 + 1) + so + 1]};
                    const half2_t m23 = {sc16[SW * (2 * s1) + so + 1], sc16[SW * (2 * s1 + 1) + so + 1]};
                    msd = __builtin_amdgcn_fdot2(p01, d01, msd, false);
                    msd = __builtin_amdgcn_fdot2(p23, d23, msd, false);
                    ms = __builtin_amdgcn_fdot2(p01, m01, ms, false);
                    ms = __builtin_amdgcn_fdot2(p23, m23, ms, false);
                }
                const h16x4 A = __builtin_bit_cast(h16x4, make_uint2(a01, a23));
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const half2_t b01 = vcode(x0, x1, r), b23 = vcode(x2, x3, r);
                    const h16x4 Bm = {b01.x, b01.y, b23.x, b23.y};
                    D[r] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, Bm, D[r], 0, 0, 0);
                }
            }
            issue(j + KS - 1, (slot + KS - 1) % KS);
            asm volatile("s_barrier" ::: "memory");
        };
        // one idle barrier (the K wave scores the first step), J work steps, idle barriers
        __syncthreads();
        // steps in groups of KS so that ring and probability slots are static
        int j = 0;
#pragma unroll 1
        for (; j + KS - 1 < J; j += KS) {
#pragma unroll
            for (int i = 0; i < KS; ++i) vstep(j + i, i);
        }
#pragma unroll
        for (int i = 0; i < KS - 1; ++i)
            if (j < J) { vstep(j, i); ++j; }
#pragma unroll 1
        for (++j; j <= Jmax; ++j) __syncthreads();
        // sum the four token groups (lanes l ^ 16, l ^ 32), each first freed of its own weight
        // scale 2^(15 + ve); offsets of all heads of the block
        const float unscale = __builtin_ldexpf(1.0f, -15 - ve);
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                D[r][c] = sum_x32(sum_x16(D[r][c] * unscale));
            }
        ms = fmaf((float)(1 << (NV - 1)), msd, ms) * (1.0f / kPScale);    // sum of p (m + o d)
        ms = sum_x32(sum_x16(ms));
        const f32x4 mh4 = {quad_bcast(ms, 0), quad_bcast(ms, 1), quad_bcast(ms, 2), quad_bcast(ms, 3)};
        wait_vmcnt<0>();                          // stages past the end, before reusing the ring
        asm volatile("" ::: "memory");
        if (tg == 0) {
            // the code scale 2^-s, the affine minimum (and the o d of the centring) and the
            // page's c_V
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int s = (NV * r) & 7;
                f32x4 v = D[r] * (1.0f / (float)(1 << (s < 10 - NV ? s : 10 - NV)));
                if (AFF_V) v += mh4;
                if (KVARN_V) v *= cvr[r];
#pragma unroll
                for (int h = 0; h < kG; ++h) S.wacc(pr)[h * kD + 32 * vblk + 8 * vj + r] = v[h];
            }
        }
        wait_vmcnt<0>();
        asm volatile("" ::: "memory");
    } else {
        // ========================= 16-bit ring chunks (binary32) =========================
        // compiled once per ring type (BF16 or binary16), chosen once per workgroup
        auto ring_role = [&](auto f16_tag) __attribute__((always_inline)) {
            constexpr bool F16 = decltype(f16_tag)::value;
            // units of 32 tokens; a step is two halves of 16 tokens (8 lanes per token pair)
            const int R = g.ring_slots;
            load_query();
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
                    const int64_t tb = sq.n_q + (int64_t)(u_first + kP * j) * kTailUnit;
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
                            const char* pk = kst + g.k.ring + (int64_t)rs * 256 + 32 * vp;
                            w[t][0] = ld_nt16(pk);
                            w[t][1] = ld_nt16(pk + 16);
                        }
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            const uint32_t ww[8] = {w[t][0].x, w[t][0].y, w[t][0].z, w[t][0].w,
                                                    w[t][1].x, w[t][1].y, w[t][1].z, w[t][1].w};
                            float kx[16];
#pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                kx[2 * i] = canon_to_f32(ww[i] & 0xFFFFu, F16);
                                kx[2 * i + 1] = canon_to_f32(ww[i] >> 16, F16);
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
                            *(float2*)&P.p[vp][16 * half + 2 * vg] = make_float2(p0, p1);
                            lsum += p0 + p1;
                        }
                    }
                    if (lane < kG) P.alpha[lane] = al;
                    __syncthreads();
                }
#pragma unroll 1
                for (; j <= Jmax; ++j) __syncthreads();
                finish_k(mh, lsum);
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
                    const int64_t tb = sq.n_q + (int64_t)(u_first + kP * j) * kTailUnit;
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
                            const char* pv = vst + g.v.ring + (int64_t)rs * 256 + 32 * vp;
                            const uint4 w0 = ld_nt16(pv), w1 = ld_nt16(pv + 16);
                            const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                vx[t][2 * i] = canon_to_f32(ww[i] & 0xFFFFu, F16);
                                vx[t][2 * i + 1] = canon_to_f32(ww[i] >> 16, F16);
                            }
                        }
                        float pp[4][2];
#pragma unroll
                        for (int h = 0; h < kG; ++h) {
                            const float2 w = *(const float2*)&P.p[h][2 * slot];
                            pp[h][0] = w.x;
                            pp[h][1] = w.y;
                        }
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
        };
        if (g.tail_f16) ring_role(std::true_type{});
        else ring_role(std::false_type{});
    }

    __syncthreads();
    float* part_out = a.partials + (int64_t)wk.slot * kPartialFloats;
    for (int i = tid; i < kG * kD; i += blockDim.x) {
        const int h = i / kD, d = i % kD;
        float M = S.wm[0][h];
#pragma unroll
        for (int p = 1; p < kP; ++p) M = fmaxf(M, S.wm[p][h]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int p = 0; p < kP; ++p) {
            const float ew = __builtin_amdgcn_exp2f(S.wm[p][h] - M);
            L += S.wl[p][h] * ew;
            A += S.wacc(p)[h * kD + d] * ew;
        }
        part_out[2 * kMaxGroup + h * kD + d] = A;
        if (d == 0) { part_out[h] = M; part_out[kMaxGroup + h] = L; }
    }
}

template <int FK, int FV>
int launch_ws_pair(const DecodeArgs& a, int n_wgs, hipStream_t st)
{
    hipLaunchKernelGGL((k_decode_ws<FK, FV>), dim3(n_wgs), dim3(kThreads), 0, st, a);
    return (int)hipGetLastError();
}

template <int FK, int FV>
int occ_ws()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_decode_ws<FK, FV>, kThreads, 0) != hipSuccess) return 0;
    return n;
}

// Key format FK against every value format of the fast kernel (op 0: launch, 1: occupancy).
template <int FK>
int ws_value_switch(int op, int fmt_v, const DecodeArgs* a, int n_wgs, hipStream_t st)
{
#define KVQ_WS_CASE(FV) \
    case FV: return op == 0 ? launch_ws_pair<FK, FV>(*a, n_wgs, st) : occ_ws<FK, FV>();
    switch (fmt_v) {
        KVQ_WS_CASE(1) KVQ_WS_CASE(2) KVQ_WS_CASE(3) KVQ_WS_CASE(4) KVQ_WS_CASE(5) KVQ_WS_CASE(6)
        KVQ_WS_CASE(7) KVQ_WS_CASE(8) KVQ_WS_CASE(9) KVQ_WS_CASE(10) KVQ_WS_CASE(11) KVQ_WS_CASE(12)
        KVQ_WS_CASE(13) KVQ_WS_CASE(14) KVQ_WS_CASE(15) KVQ_WS_CASE(16) KVQ_WS_CASE(17) KVQ_WS_CASE(18)
        KVQ_WS_CASE(19) KVQ_WS_CASE(20) KVQ_WS_CASE(21) KVQ_WS_CASE(22) KVQ_WS_CASE(23) KVQ_WS_CASE(24)
    default: return op == 0 ? (int)hipErrorInvalidValue : 0;
    }
#undef KVQ_WS_CASE
}

}  // namespace

}  // namespace kvq
