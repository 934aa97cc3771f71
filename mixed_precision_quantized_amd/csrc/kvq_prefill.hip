// kvq_prefill.hip -- causal chunked-prefill attention over the mixed-precision cache, gfx950.
//
// After a chunk of n_new tokens has been appended, query i of the chunk (position
// p = n - n_new + i) attends to the tokens t <= p as the cache holds them: dequantized rows
// below n_q, BF16 ring rows above.  Prefill is measured on its own, apart from decode ("Форк
// beellama и KV-кванты kvarn на длинном контексте", the section on how to compare builds);
// unlike single-token decode it is a dense contraction (every key meets every query of the
// chunk), so it runs on the matrix cores:
//
//   workgroup = (KV head, 32 query positions, key split): four waves, one per query head of
//   the KV head's group, each owning 32 queries; the raw bytes of each 32-key block are
//   loaded straight to LDS two blocks ahead and unpacked to binary16 one block ahead;
//   per 32-key block each wave computes
//   S^T = K Q^T (32 keys x 32 queries, v_mfma_f32_32x32x16_f16: a lane holds one query and
//   16 of the keys, so the softmax of a query is a reduction over registers and one lane
//   pair), the online softmax, and O^T += V^T P^T (128 dims x 32 queries, four 32x32 tiles).
//
// Precision.  Keys enter as their exact centred codes (u - o, or u for affine codes: small
// integers, exact in binary16); the block scale d of each (token, block) is applied to the
// binary32 product of that block's 32 dims, and the affine minimum m as m * sum(q) of the
// block, so the keys are used exactly.  (Rounding dequantized keys to binary16 would not do:
// keys with 15x outlier channels reach |k| ~ 800, where binary16 keeps 0.25 absolute.)
// 16-bit key rows (ring, bf16 format) enter as k 2^-s with the power of two s per (token,
// block) that puts the block's largest |k| in [2^14, 2^15), and d = 2^s: exact for every
// bf16 value of the block down to 2^-24 of its maximum, beyond binary16's range included.
// The query enters as two binary16 terms, q 2^-sq = hi + lo, one MFMA each (sq per query,
// its largest |q| in [2^7, 2^8); the scores are scaled back by 2^sq): one rounding of q
// alone cost up to 1.9e-3 of the output on the 64k block-format workload.  Values enter as
// binary16 v 2^sv, with one sv per workgroup taken from a bound on |v| over its split (read
// from the block scales and channel scales, or from the 16-bit rows, before the loop) so
// that |v 2^sv| < 2^15; the probabilities as binary16 2^15 p.  Neither then overflows, and
// neither loses small values to the binary16 subnormals, whatever the values' magnitude;
// the split's accumulator is scaled back by 2^-(15 + sv).
//
// KVarN (either inner quantizer): keys are scored in the rotated domain against
// q' = H q / 128.  The page's key channel scale goes to the key side: c (u - o) is exact in
// binary32 and is held as two exact binary16 terms hi + lo (11 and at most 8 significant
// bits), scored as q'_hi hi + q'_lo hi + q'_hi lo (q'_lo lo is below 2^-20 of the term);
// no per-page query operand is built.  Over affine blocks the minimum term takes
// m sum_j q'_j c_j per page.  Values accumulate in the rotated domain and are rotated back
// once in the merge (quantized and ring blocks never share a split, so each split is in one
// domain).
#include "kvq_device.h"

namespace kvq {

namespace {

constexpr int kG = 4;
constexpr float kNeg = -1.0e30f;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct alignas(16) PfLds {
    _Float16 kc[kPfKB][kD + 8];     // key codes (or exact values), token-major; +8: bank spread
    _Float16 kl[kPfKB][kD + 8];     // paged keys: c (u - o) = kc + kl, both binary16-exact
    _Float16 vt[kD][kPfKB + 8];     // dequantized values, dim-major
    float dk[4][kPfKB];             // key block scales [block][token] (1 for exact rows)
    float mk[4][kPfKB];             // key block minima (affine codes)
    float ck[kD];                   // KVarN key channel scales of the block's page
    int kscaled[4];                 // per key-unpacking wave: some 16-bit row was range-scaled
};

// The two halves of the wave exchanged by v_permlane32_swap (no LDS round trip): with both
// operands x, one result holds x of lanes 0-31 in both halves and the other x of lanes
// 32-63, so their maximum or sum is that of x with the lane l ^ 32 in every lane.
__device__ __forceinline__ float max_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ const char* pf_stream(const CacheGeom& g, int seq, int layer, int head, int isv)
{
    const int64_t unit = ((int64_t)seq * g.n_layers + layer) * g.n_kv_heads + head;
    return g.base + unit * g.unit_bytes + (isv ? g.v_offset : 0);
}

// Staging of one 32-token block.  Its raw bytes (codes, scales, channel scales, or BF16
// rows) are loaded straight to LDS by buffer loads two blocks ahead of use (no registers,
// the latency overlaps the compute of two blocks); one block ahead, the waves unpack them
// into the binary16 operand buffers.
template <bool BIG>
struct alignas(16) PfRawL {
    static constexpr int kRows = BIG ? 8192 : 4096;    // BF16 rows (32 x 256 B), or 32 rows of 16 N <= 128 B
    uint8_t k[kRows];
    uint8_t v[kRows];
    uint8_t ks[512];       // block-scale rows (8 or 16 B per token)
    uint8_t vs[512];
    uint16_t kch[128];     // KVarN channel scales of the block's page
    uint16_t vch[128];
};

typedef __amdgpu_buffer_rsrc_t pf_rsrc_t;
__device__ __forceinline__ pf_rsrc_t pf_rsrc(const void* p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
// lane l copies 16 bytes from the resource at voff to lds + 16 l (reads past the resource's
// size return zero); the wait is explicit (pf_wait_vm0).  M0 is set in the same block.
__device__ __forceinline__ void pf_dma16(pf_rsrc_t r, int voff, const void* lds)
{
    const uint32_t la = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds\n\ts_nop 0"
                 :: "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(la)) : "memory", "m0");
}
__device__ __forceinline__ void pf_wait_vm0()
{
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0) only
}

// One stream's bases and the issue of one block's loads into R (every wave: 2 x 64 chunks
// per stream; chunk c of a block = bytes 16 c of its rows).  Quantized rows: a buffer
// resource per block, from a 64-bit base (rows past the block's valid ones read as zero),
// so no offset grows with the context; ring rows: one resource over the ring.
struct PfStream {
    pf_rsrc_t ring_rows;    // ring streams
    const char* codes;      // quantized streams: rows, block scales, channel scales
    const char* scales;
    const char* chan;
    int rb, sb;             // code (or BF16) bytes per row, scale bytes per row
    bool ring;
};
__device__ __forceinline__ PfStream pf_stream_rsrc(const PrefillArgs& a, const char* st, const StreamLayout& Ls,
                                                   int fmt, bool quant)
{
    PfStream S;
    const bool exact = fkind(fmt) == KIND_BF16;
    S.ring = !quant;
    S.rb = quant && !exact ? 16 * fbits(fmt) : 256;
    S.sb = kind_affine(fkind(fmt)) ? 16 : 8;
    S.codes = st + Ls.codes;
    S.scales = st + Ls.scales;
    S.chan = st + (Ls.cscale >= 0 ? Ls.cscale : 0);
    S.ring_rows = pf_rsrc(st + Ls.ring, quant ? 0 : a.g.ring_slots * 256);
    (void)exact;
    return S;
}

// NW waves: 4 load both streams, 8 split them (waves 0-3 keys, 4-7 values).
template <int KK, int KV, bool RING, bool BIG, int NW>
__device__ __forceinline__ void pf_dma(PfRawL<BIG>& R, const PrefillArgs& a, const PfStream& SK, const PfStream& SV,
                                       int64_t tb, int nt, int wave_, int lane)
{
    const int wave = wave_ & 3;
    auto stream = [&](const PfStream& S, bool coded, bool kvarn, uint8_t* dst, uint8_t* sdst, uint16_t* cdst,
                      int swave, int cwave) {
        if (!RING) {
            // the block's 2 rb chunks of 16 B (256 for codes of 8 bits or less: one per thread)
            const pf_rsrc_t rows = pf_rsrc(S.codes + tb * S.rb, nt * S.rb);
#pragma unroll
            for (int i = 0; i < (BIG ? 2 : 1); ++i) {
                const int c0 = 64 * (wave + 4 * i);
                if (c0 + lane < 2 * S.rb) pf_dma16(rows, 16 * (c0 + lane), dst + 16 * c0);
            }
            if (coded && wave == swave && lane < 32)
                pf_dma16(pf_rsrc(S.scales + tb * S.sb, nt * S.sb), 16 * lane, sdst);
            if (kvarn && wave == cwave && lane < 16)
                pf_dma16(pf_rsrc(S.chan + (tb / kPage) * 256, 256), 16 * lane, cdst);
        } else {
            // ring rows: slot (t mod R); rows past nt read past the resource (zero)
            const int R = a.g.ring_slots;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int c0 = 64 * (wave + 4 * i), c = c0 + lane, r = c >> 4;
                const int voff = r < nt ? (int)((tb + r) % R) * 256 + 16 * (c & 15) : R * 256;
                pf_dma16(S.ring_rows, voff, dst + 16 * c0);
            }
        }
    };
    if (NW == 4 || wave_ < 4) stream(SK, KK != KIND_BF16, kind_paged(KK), R.k, R.ks, R.kch, 0, 2);
    if (NW == 4 || wave_ >= 4) stream(SV, KV != KIND_BF16, kind_paged(KV), R.v, R.vs, R.vch, 1, 3);
}

// 16 N-bit codes of part `part` of a row held at lds row (dword aligned)
template <int N>
__device__ __forceinline__ void unpack16(const uint8_t* row, int part, uint32_t (&u)[16])
{
    const int b0 = 2 * N * part, fd = b0 >> 2, sh0 = 8 * (b0 & 3);
    const uint32_t* p = (const uint32_t*)row + fd;
    uint32_t w[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) w[i] = (32 * i < sh0 + 16 * N) ? p[i] : 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int bit = sh0 + N * e, wi = bit >> 5, sh = bit & 31;
        uint32_t v = w[wi] >> sh;
        if (sh + N > 32) v |= w[wi + 1] << (32 - sh);
        u[e] = v & ((1u << N) - 1u);
    }
}
__device__ __forceinline__ void unpack16_rt(int N, const uint8_t* row, int part, uint32_t (&u)[16])
{
    switch (N) {
    case 2: unpack16<2>(row, part, u); break;
    case 3: unpack16<3>(row, part, u); break;
    case 4: unpack16<4>(row, part, u); break;
    case 5: unpack16<5>(row, part, u); break;
    case 6: unpack16<6>(row, part, u); break;
    default: unpack16<8>(row, part, u); break;
    }
}

// Codes of 2, 4 or 8 bits: the 16 codes of part `part` of a row as eight binary16 pairs
// (dims 2i, 2i + 1) holding u - off exactly.  The byte that holds a pair is copied to both
// halves of a word (v_perm); a mask keeps one code per half, at bit 0 in the low half and
// at bit s in the high one, under the exponent bits of 1024 (ulp 1 in [1024, 2048)); one
// binary16 fma then scales by 2^-s and subtracts 1024 + off.  Every step is exact.
template <int N>
__device__ __forceinline__ void codes_h2(const uint8_t* row, int part, float off, h2 (&o)[8])
{
    static_assert(N == 2 || N == 4 || N == 8, "2-, 4- or 8-bit codes");
    const uint32_t* p = (const uint32_t*)(row + 2 * N * part);
    const _Float16 a0 = (_Float16)(-1024.0f - off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t x;
        h2 sc, ad;
        if constexpr (N == 8) {
            // bytes 2i, 2i + 1 under the exponent byte 0x64
            const uint32_t b = 2 * (i & 1);
            x = __builtin_amdgcn_perm(0x64646464u, p[i >> 1], b | (4u << 8) | ((b + 1) << 16) | (4u << 24));
            sc = (h2){(_Float16)1.0f, (_Float16)1.0f};
            ad = (h2){a0, a0};
        } else if constexpr (N == 4) {
            const uint32_t b = i & 3;
            x = __builtin_amdgcn_perm(p[i >> 2], p[i >> 2], b * 0x01010101u);
            x = (x & 0x00F0000Fu) | 0x64006400u;
            sc = (h2){(_Float16)1.0f, (_Float16)0.0625f};
            ad = (h2){a0, (_Float16)(-64.0f - off)};
        } else {
            const uint32_t b = (i >> 1) & 3;
            x = __builtin_amdgcn_perm(p[i >> 3], p[i >> 3], b * 0x01010101u);
            if (i & 1) {
                x = (x & 0x00C00030u) | 0x64006400u;
                sc = (h2){(_Float16)0.0625f, (_Float16)0.015625f};
                ad = (h2){(_Float16)(-64.0f - off), (_Float16)(-16.0f - off)};
            } else {
                x = (x & 0x000C0003u) | 0x64006400u;
                sc = (h2){(_Float16)1.0f, (_Float16)0.25f};
                ad = (h2){a0, (_Float16)(-256.0f - off)};
            }
        }
        o[i] = __builtin_elementwise_fma(__builtin_bit_cast(h2, x), sc, ad);
    }
}
__device__ __forceinline__ bool codes_h2_rt(int N, const uint8_t* row, int part, float off, h2 (&o)[8])
{
    switch (N) {
    case 2: codes_h2<2>(row, part, off, o); return true;
    case 4: codes_h2<4>(row, part, off, o); return true;
    case 8: codes_h2<8>(row, part, off, o); return true;
    default: return false;
    }
}

// Unpack a raw block into the operand buffers.  Thread tid (0..255): token r, dims 16 pp ..
// of the keys (PART 1), the values (PART 2) or both (PART 0); r = tid >> 3, pp = tid & 7,
// except for values alone (r = tid & 31, pp = tid >> 5).
template <int KK, int KV, bool RING, bool BIG, int PART>
__device__ __forceinline__ void pf_unpack(PfLds& L, const PfRawL<BIG>& R, const PrefillArgs& a, int nt, bool quant, int tid,
                                          float vmul)
{
    constexpr bool DK = PART != 2, DV = PART != 1;
    const CacheGeom& g = a.g;
    // values alone: token-fastest threads, so that the dim-major value stores of a wave fall
    // on consecutive halves of a row (16-way bank conflicts with dims-fastest threads)
    const int r = PART == 2 ? (tid & 31) : (tid >> 3), pp = PART == 2 ? (tid >> 5) : (tid & 7), b = pp >> 1;
    const bool valid = r < nt;
    float kx[16], vx[16];
    float d = 1.0f, m = 0.0f;
    bool kdone = false;     // keys already stored (2-, 4- and 8-bit codes in binary16 pairs)
    if (DK && quant && KK != KIND_BF16) {
        if (kind_affine(KK)) {
            const uint32_t dm = *(const uint32_t*)(R.ks + r * 16 + 4 * b);
            d = fp16_to_f32(dm & 0xFFFFu);
            m = fp16_to_f32(dm >> 16);
        } else {
            d = fp16_to_f32(*(const uint16_t*)(R.ks + r * 8 + 2 * b));
        }
        const int N = fbits(g.fmt_k);
        h2 uo[8];
        // (not for kvarnN_1 streams: their kernel is the one short of registers, and the
        // binary32 route spills less there)
        if (KK != KIND_KVARN1 && codes_h2_rt(N, R.k + r * 16 * N, pp, kind_affine(KK) ? 0.0f : (float)(1 << (N - 1)), uo)) {
            kdone = true;
            uint32_t w[8], wl[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (kind_paged(KK) && !RING) {
                    // c (u - o) rounded to binary16, and its exact remainder: the same two
                    // terms as the binary32 route below (the product is exact there)
                    const h2 c2 = ((const h2*)R.kch)[8 * pp + i];
                    const h2 hi = uo[i] * c2;
                    const h2 lo = __builtin_elementwise_fma(uo[i], c2, -hi);
                    w[i] = valid ? __builtin_bit_cast(uint32_t, hi) : 0u;
                    wl[i] = valid ? __builtin_bit_cast(uint32_t, lo) : 0u;
                } else {
                    w[i] = valid ? __builtin_bit_cast(uint32_t, uo[i]) : 0u;
                    wl[i] = 0u;
                }
            }
            uint4* dst = (uint4*)&L.kc[r][16 * pp];
            dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
            dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
            if (kind_paged(KK) && !RING) {
                uint4* dl = (uint4*)&L.kl[r][16 * pp];
                dl[0] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
                dl[1] = make_uint4(wl[4], wl[5], wl[6], wl[7]);
            }
        }
    }
    if (!DK || kdone) {
    } else if (quant && KK != KIND_BF16) {
        const int N = fbits(g.fmt_k);
        uint32_t u[16];
        unpack16_rt(N, R.k + r * 16 * N, pp, u);
        const float off = kind_affine(KK) ? 0.0f : (float)(1 << (N - 1));
#pragma unroll
        for (int e = 0; e < 16; ++e) kx[e] = (float)u[e] - off;
        if (kind_paged(KK) && !RING) {
            // the page's key channel scale on the key side: c (u - o) is exact in binary32
            // (11 + N significant bits) and splits into two exact binary16 terms
#pragma unroll
            for (int e = 0; e < 16; ++e) kx[e] *= fp16_to_f32(R.kch[16 * pp + e]);
        }
    } else {
        const uint4* q = (const uint4*)(R.k + r * 256 + 32 * pp);
        const uint4 x0 = q[0], x1 = q[1];
        const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kx[2 * i] = canon_to_f32(w[i] & 0xFFFFu, !quant && g.tail_f16);
            kx[2 * i + 1] = canon_to_f32(w[i] >> 16, !quant && g.tail_f16);
        }
        // a block whose largest |k| (its other half is in the neighbouring lane) lies outside
        // [2^-10, 2^15) is scaled to [2^14, 2^15): binary16 then holds its large elements
        // without overflow and its small ones to 2^-25 of the block maximum or better, as
        // it does unscaled inside that range
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(kx[e]));
        amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(amax), 0xB1, 0xF, 0xF, false)));
        if (amax > 0.0f && !(amax >= 0x1p-10f && amax < 32768.0f)) {
            const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
            const int sh = min(126, max(-126, (ex == 0 ? 1 : ex) - 127 - 14));
            const float f = __builtin_ldexpf(1.0f, -sh);
#pragma unroll
            for (int e = 0; e < 16; ++e) kx[e] *= f;
            d = __builtin_ldexpf(1.0f, sh);
        }
    }
    // values: the power of two vmul enters with the block scale and minimum (exact: the
    // results are those of scaling afterwards, nothing here leaves the binary32 range)
    if (!DV) {
    } else if (quant && KV != KIND_BF16) {
        const int N = fbits(g.fmt_v);
        const float off = kind_affine(KV) ? 0.0f : (float)(1 << (N - 1));
        float dv, mv = 0.0f;
        if (kind_affine(KV)) {
            const uint32_t dm = *(const uint32_t*)(R.vs + r * 16 + 4 * b);
            dv = fp16_to_f32(dm & 0xFFFFu) * vmul;
            mv = fp16_to_f32(dm >> 16) * vmul;
        } else {
            dv = fp16_to_f32(*(const uint16_t*)(R.vs + r * 8 + 2 * b)) * vmul;
        }
        h2 uo[8];
        if (KV != KIND_KVARN1 && codes_h2_rt(N, R.v + r * 16 * N, pp, off, uo)) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                vx[2 * i] = (float)uo[i].x;
                vx[2 * i + 1] = (float)uo[i].y;
            }
        } else {
            uint32_t u[16];
            unpack16_rt(N, R.v + r * 16 * N, pp, u);
#pragma unroll
            for (int e = 0; e < 16; ++e) vx[e] = (float)u[e] - off;
        }
        // affine: d u + m in one rounding; symmetric: (u - o) d, exact
#pragma unroll
        for (int e = 0; e < 16; ++e) vx[e] = kind_affine(KV) ? fmaf(dv, vx[e], mv) : vx[e] * dv;
        if (kind_paged(KV)) {
#pragma unroll
            for (int e = 0; e < 16; ++e) vx[e] *= fp16_to_f32(R.vch[16 * pp + e]);
        }
    } else {
        const uint4* q = (const uint4*)(R.v + r * 256 + 32 * pp);
        const uint4 x0 = q[0], x1 = q[1];
        const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            vx[2 * i] = canon_to_f32(w[i] & 0xFFFFu, !quant && g.tail_f16) * vmul;
            vx[2 * i + 1] = canon_to_f32(w[i] >> 16, !quant && g.tail_f16) * vmul;
        }
    }
    if (!valid) {
#pragma unroll
        for (int e = 0; e < 16; ++e) { kx[e] = 0.0f; vx[e] = 0.0f; }
    }
    if (DK && !kdone) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const h2 v = {(_Float16)kx[2 * i], (_Float16)kx[2 * i + 1]};
            w[i] = __builtin_bit_cast(uint32_t, v);
        }
        uint4* dst = (uint4*)&L.kc[r][16 * pp];
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        if (kind_paged(KK) && !RING) {
            // low parts: c (u - o) - hi, at most 8 significant bits
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const h2 hv = __builtin_bit_cast(h2, w[i]);
                const h2 v = {(_Float16)(kx[2 * i] - (float)hv.x), (_Float16)(kx[2 * i + 1] - (float)hv.y)};
                w[i] = __builtin_bit_cast(uint32_t, v);
            }
            uint4* dl = (uint4*)&L.kl[r][16 * pp];
            dl[0] = make_uint4(w[0], w[1], w[2], w[3]);
            dl[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
    }
    if (DV) {
#pragma unroll
        for (int e = 0; e < 16; ++e) L.vt[16 * pp + e][r] = (_Float16)vx[e];
    }
    if (DK && (pp & 1) == 0) {
        L.dk[b][r] = d;
        L.mk[b][r] = m;
    }
    if (DK) {
        // 16-bit rows: whether any row of the block took a scale (else the scores skip dk)
        const bool any = __builtin_amdgcn_ballot_w64(d != 1.0f) != 0;
        if ((tid & 63) == 0) L.kscaled[(tid >> 6) & 3] = any ? 1 : 0;
    }
    if (DK && kind_paged(KK) && !RING && tid < kD) L.ck[tid] = fp16_to_f32(R.kch[tid]);
}

// RING: the kernel of the ring (16-bit) splits, else of the quantized splits.  The
// kernel runs NT = 2 query tiles per workgroup: 8 waves (two per SIMD: at one the kernel
// is latency-bound) share each staged and unpacked block.  The quantized kernel's raw
// staging holds code rows only (at most 4 KB per stream); BIG staging holds BF16 rows (the
// ring splits, bf16-format streams).  kvarnN_1 keys spill ~230 B per lane within the 256
// registers and are still twice as fast as with one tile of 4 waves.
template <int KK, int KV, bool RING, bool BIG = RING || KK == KIND_BF16 || KV == KIND_BF16, int NT = 2>
__global__ __launch_bounds__(256 * NT, 1) void k_prefill(PrefillArgs a)
{
    // Wave w computes query head w % 4 of the group for the 32 queries of tile w / 4 and,
    // with the others, stages the blocks: block i + 2 is loaded to raw LDS and block i + 1
    // unpacked while block i is computed; one barrier per block.
    __shared__ PfLds L[2];
    __shared__ PfRawL<BIG> RW[2];
    __shared__ float vbnd[2][4 * NT];      // per wave: bound of |v| over the split, and of |c_V|
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int S = a.splits_q + a.splits_t;
    const int SS = RING ? a.splits_t : a.splits_q;                   // splits of this kernel
    const int tiles_g = (a.tiles + NT - 1) / NT;                     // tile groups
    const int sp = (RING ? a.splits_q : 0) + blockIdx.x % SS;
    const int tg = (blockIdx.x / SS) % tiles_g;
    const int head = blockIdx.x / (SS * tiles_g);
    const int tile = NT * tg + (wave >> 2);                          // this wave's tile
    constexpr bool quant = !RING;
    const CacheGeom& g = a.g;
    const char* kst = pf_stream(g, a.seq, a.layer, head, 0);
    const char* vst = pf_stream(g, a.seq, a.layer, head, 1);
    // the workgroup's last query
    const int64_t pos_max = a.n - a.n_new + min(kPfQ * NT * (tg + 1), a.n_new) - 1;

    // ---- key range of the split (32-token blocks of the quantized or the ring region) ------
    const int64_t r0 = quant ? 0 : a.n_q, r1 = quant ? a.n_q : a.n;
    const int bps = RING ? a.bps_t : a.bps;
    const int blk0 = (quant ? sp : sp - a.splits_q) * bps;
    const int nblk = (int)((r1 - r0 + kPfKB - 1) / kPfKB);
    const int blk1 = min(blk0 + bps, nblk);
    // causal: no key after the workgroup's last query is seen
    const int blk_end = pos_max < r0 ? blk0 : (int)min<int64_t>(blk1, (pos_max - r0) / kPfKB + 1);
    const int nb = max(0, blk_end - blk0);
    auto tb_of = [&](int i) { return r0 + (int64_t)(blk0 + i) * kPfKB; };
    auto nt_of = [&](int i) { return (int)min<int64_t>(kPfKB, r1 - tb_of(i)); };

    // ================================ compute waves ================================
    const int h = wave & 3;                                          // query head of the group
    const int j = lane & 31, hh = lane >> 5;
    const int qi = kPfQ * tile + j;                                  // query index in the chunk
    const bool qvalid = qi < a.n_new;
    const int64_t pos = a.n - a.n_new + (qvalid ? qi : a.n_new - 1);
    const int64_t pos_min = a.n - a.n_new + kPfQ * tile;             // the tile's first query
    constexpr bool kv_k = kind_paged(KK) && !RING;

    // ---- query: the lane's 64 dims {16 idx + 8 hh + c}, log2 domain, as hi + lo binary16 ----
    h8 qb[8], ql[8];                 // the query operand (paged keys: H q / 128) = (qb + ql) qmul
    float qmul = 1.0f;
    {
        float qf[8][8];
        const int64_t base = ((int64_t)(qvalid ? qi : 0) * g.n_q_heads + head * kG + h) * kD;
#pragma unroll
        for (int idx = 0; idx < 8; ++idx)
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int64_t e = base + 16 * idx + 8 * hh + c;
                const float v = a.q_dtype ? ((const float*)a.q)[e] : bf16_to_f32(((const uint16_t*)a.q)[e]);
                qf[idx][c] = qvalid ? v * a.scale_log2 : 0.0f;
            }
        if (kv_k) {
            // H q / 128: spans 1, 2, 4 (c) and 16, 32, 64 (idx) in the lane, 8 across the pair
#pragma unroll
            for (int idx = 0; idx < 8; ++idx)
#pragma unroll
                for (int sp2 = 1; sp2 < 8; sp2 <<= 1)
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        if ((c & sp2) == 0) {
                            const float x = qf[idx][c], y = qf[idx][c + sp2];
                            qf[idx][c] = x + y;
                            qf[idx][c + sp2] = x - y;
                        }
#pragma unroll
            for (int s2 = 1; s2 < 8; s2 <<= 1)
#pragma unroll
                for (int idx = 0; idx < 8; ++idx)
                    if ((idx & s2) == 0)
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            const float x = qf[idx][c], y = qf[idx + s2][c];
                            qf[idx][c] = x + y;
                            qf[idx + s2][c] = x - y;
                        }
#pragma unroll
            for (int idx = 0; idx < 8; ++idx)
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float y = __shfl_xor(qf[idx][c], 32);
                    qf[idx][c] = (hh ? y - qf[idx][c] : qf[idx][c] + y) * (1.0f / 128.0f);
                }
        }
        // power of two of the query: its largest |q| (over the lane pair) to [2^7, 2^8)
        float amax = 0.0f;
#pragma unroll
        for (int idx = 0; idx < 8; ++idx)
#pragma unroll
            for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(qf[idx][c]));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        if (amax > 0.0f) {
            const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
            const int sq = min(126, max(-126, (ex == 0 ? 1 : ex) - 127 - 7));
            const float f = __builtin_ldexpf(1.0f, -sq);
            qmul = __builtin_ldexpf(1.0f, sq);
#pragma unroll
            for (int idx = 0; idx < 8; ++idx)
#pragma unroll
                for (int c = 0; c < 8; ++c) qf[idx][c] *= f;
        }
#pragma unroll
        for (int idx = 0; idx < 8; ++idx)
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const _Float16 hi = (_Float16)qf[idx][c];
                qb[idx][c] = hi;
                ql[idx][c] = (_Float16)(qf[idx][c] - (float)hi);
            }
    }
    float qsum[4];
    auto make_qsum = [&]() {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c)
                s += ((float)qb[2 * b][c] + (float)ql[2 * b][c]) + ((float)qb[2 * b + 1][c] + (float)ql[2 * b + 1][c]);
            qsum[b] = s + __shfl_xor(s, 32);
        }
    };
    if (KK == KIND_Q1) make_qsum();
    // paged keys over affine blocks: the minimum term m sum_j q'_j c_j takes the block sums
    // of the rotated query times the page's key channel scales, per page
    auto page_qsum = [&](const PfLds& B) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float s = 0.0f;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int idx = 2 * b + k2;
                    s = fmaf((float)qb[idx][c] + (float)ql[idx][c], B.ck[16 * idx + 8 * hh + c], s);
                }
            qsum[b] = s + __shfl_xor(s, 32);
        }
    };

    float mrun = kNeg, lrun = 0.0f;
    f32x16 O[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[b][r] = 0.0f;
    int64_t page = -1;
    // key rows of this lane in the 32x32 accumulators: i(r) = 8 (r / 4) + 4 hh + r % 4
    auto compute = [&](const PfLds& B, int64_t tb, int nt) __attribute__((always_inline)) {
        if (kv_k && KK == KIND_KVARN1 && tb / kPage != page) {
            page = tb / kPage;
            page_qsum(B);
        }
        // S^T: keys x queries
        f32x16 Sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) Sacc[r] = 0.0f;
        constexpr bool aff_k = !RING && kind_affine(KK);
        constexpr bool exact_k = RING || KK == KIND_BF16;
        if (exact_k && !(B.kscaled[0] | B.kscaled[1] | B.kscaled[2] | B.kscaled[3])) {
            // 16-bit rows, none scaled: one accumulator over the four blocks
            f32x16 T;
#pragma unroll
            for (int r = 0; r < 16; ++r) T[r] = 0.0f;
#pragma unroll
            for (int idx = 0; idx < 8; ++idx) {
                const h8 A = *(const h8*)&B.kc[j][16 * idx + 8 * hh];
                T = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, qb[idx], T, 0, 0, 0);
                T = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, ql[idx], T, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Sacc[r] = T[r];
        } else
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f32x16 T;
#pragma unroll
            for (int r = 0; r < 16; ++r) T[r] = 0.0f;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int idx = 2 * b + k2;
                const h8 A = *(const h8*)&B.kc[j][16 * idx + 8 * hh];
                T = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, qb[idx], T, 0, 0, 0);
                T = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, ql[idx], T, 0, 0, 0);
                if (kv_k) {
                    // low key term against the high query term (lo x lo is below 2^-20)
                    const h8 Al = *(const h8*)&B.kl[j][16 * idx + 8 * hh];
                    T = __builtin_amdgcn_mfma_f32_32x32x16_f16(Al, qb[idx], T, 0, 0, 0);
                }
            }
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 dd = *(const float4*)&B.dk[b][8 * r4 + 4 * hh];
                const float dv[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) Sacc[4 * r4 + c] = fmaf(dv[c], T[4 * r4 + c], Sacc[4 * r4 + c]);
                if (aff_k) {
                    const float4 mm = *(const float4*)&B.mk[b][8 * r4 + 4 * hh];
                    const float mv[4] = {mm.x, mm.y, mm.z, mm.w};
#pragma unroll
                    for (int c = 0; c < 4; ++c) Sacc[4 * r4 + c] = fmaf(mv[c], qsum[b], Sacc[4 * r4 + c]);
                }
            }
        }
        // The scores are Sacc qmul (qmul a power of two, so the product is exact and the
        // maximum may be taken before it).  Masked blocks: rows past the block's end, and keys
        // later than the query (only blocks that reach the tile's first query or end early;
        // unused query slots are never read back).
        float mx = kNeg, mn;
        float ps = 0.0f;
        float p[16];
        if (nt < kPfKB || tb + kPfKB - 1 > pos_min) {
            const int lim = (int)min<int64_t>(nt - 1, pos - tb);      // last visible row
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 8 * (r >> 2) + 4 * hh + (r & 3);
                Sacc[r] = i > lim ? kNeg : Sacc[r] * qmul;
                mx = fmaxf(mx, Sacc[r]);
            }
            mx = max_xor32(mx);
            mn = fmaxf(mrun, mx);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = Sacc[r] > 0.5f * kNeg ? __builtin_amdgcn_exp2f(Sacc[r] - mn) : 0.0f;
                ps += p[r];
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, Sacc[r]);
            mx = max_xor32(mx) * qmul;
            mn = fmaxf(mrun, mx);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = __builtin_amdgcn_exp2f(fmaf(Sacc[r], qmul, -mn));
                ps += p[r];
            }
        }
        const float al = __builtin_amdgcn_exp2f(mrun - mn);
        ps = sum_xor32(ps);
        lrun = fmaf(lrun, al, ps);
        mrun = mn;
        if (__builtin_amdgcn_ballot_w64(al != 1.0f)) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) O[b][r] *= al;
        }
        // O^T += V^T P^T: K slot 8 hh + c of MFMA k2 is key 16 k2 + 8 (c / 4) + 4 hh + c % 4,
        // which is accumulator register 8 k2 + c of this lane
        h8 pb[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int c = 0; c < 8; ++c) pb[k2][c] = (_Float16)(p[8 * k2 + c] * 32768.0f);
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const _Float16* row = &B.vt[32 * b + j][0];
                const uint2 lo = *(const uint2*)(row + 16 * k2 + 4 * hh);
                const uint2 hi = *(const uint2*)(row + 16 * k2 + 8 + 4 * hh);
                const h8 A = __builtin_bit_cast(h8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                O[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, pb[k2], O[b], 0, 0, 0);
            }
    };
    const PfStream SK = pf_stream_rsrc(a, kst, g.k, g.fmt_k, quant), SV = pf_stream_rsrc(a, vst, g.v, g.fmt_v, quant);
    if (nb > 0) pf_dma<KK, KV, RING, BIG, 4 * NT>(RW[0], a, SK, SV, tb_of(0), nt_of(0), wave, lane);
    if (nb > 1) pf_dma<KK, KV, RING, BIG, 4 * NT>(RW[1], a, SK, SV, tb_of(1), nt_of(1), wave, lane);
    // ---- a bound on |v| over the split's value rows, read while the first blocks load ------
    // quantized: |d| 2^(N-1) (symmetric) or |d| (2^N - 1) + |m| (affine) per (token, block),
    // times the largest |c_V| of the split's pages; 16-bit rows: their largest |v|
    {
        float vb = 0.0f, cb = 0.0f;
        if (nb > 0) {
            const int64_t t0 = tb_of(0), t1 = tb_of(nb - 1) + nt_of(nb - 1);
            const int nthr = 256 * NT;
            if (quant && KV != KIND_BF16) {
                const int N = fbits(g.fmt_v);
                const char* vsc = vst + g.v.scales;
                if (kind_affine(KV)) {
                    const float top = (float)((1 << N) - 1);
                    for (int64_t t = t0 + tid; t < t1; t += nthr) {
                        const uint4 w = *(const uint4*)(vsc + t * 16);
                        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            vb = fmaxf(vb, fmaf(fabsf(fp16_to_f32(ww[i] & 0xFFFFu)), top, fabsf(fp16_to_f32(ww[i] >> 16))));
                    }
                } else {
                    const float off = (float)(1 << (N - 1));
                    for (int64_t t = t0 + tid; t < t1; t += nthr) {
                        const uint2 w = *(const uint2*)(vsc + t * 8);
                        const float d4 = fmaxf(fmaxf(fabsf(fp16_to_f32(w.x & 0xFFFFu)), fabsf(fp16_to_f32(w.x >> 16))),
                                               fmaxf(fabsf(fp16_to_f32(w.y & 0xFFFFu)), fabsf(fp16_to_f32(w.y >> 16))));
                        vb = fmaxf(vb, d4 * off);
                    }
                }
                if (kind_paged(KV)) {
                    const uint16_t* ch = (const uint16_t*)(vst + g.v.cscale);
                    for (int64_t i = (t0 / kPage) * kD + tid; i < ((t1 - 1) / kPage + 1) * kD; i += nthr)
                        cb = fmaxf(cb, fabsf(fp16_to_f32(ch[i])));
                }
            } else {
                const bool f16r = !quant && g.tail_f16;
                for (int64_t i = t0 * 16 + tid; i < t1 * 16; i += nthr) {
                    const int64_t t = i >> 4;
                    const char* row = quant ? vst + g.v.codes + t * 256 : vst + g.v.ring + (t % g.ring_slots) * 256;
                    const uint4 w = *(const uint4*)(row + 16 * (i & 15));
                    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        vb = fmaxf(vb, fmaxf(fabsf(canon_to_f32(ww[k] & 0xFFFFu, f16r)), fabsf(canon_to_f32(ww[k] >> 16, f16r))));
                }
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            vb = fmaxf(vb, __shfl_xor(vb, o));
            cb = fmaxf(cb, __shfl_xor(cb, o));
        }
        if (lane == 0) {
            vbnd[0][wave] = vb;
            vbnd[1][wave] = cb;
        }
    }
    pf_wait_vm0();
    __syncthreads();
    // value exponent sv: the bound times 2^sv in [2^14, 2^15)
    float vmul = 1.0f, ounscale = 1.0f / 32768.0f;
    {
        float vmax = 0.0f, cmax = 0.0f;
#pragma unroll
        for (int w = 0; w < 4 * NT; ++w) {
            vmax = fmaxf(vmax, vbnd[0][w]);
            cmax = fmaxf(cmax, vbnd[1][w]);
        }
        const float bound = (quant && kind_paged(KV)) ? vmax * cmax : vmax;
        if (bound > 0.0f) {
            const int ex = (int)((__float_as_uint(bound) >> 23) & 0xFFu);
            const int sv = min(126, max(-126, 14 - ((ex == 0 ? 1 : ex) - 127)));
            vmul = __builtin_ldexpf(1.0f, sv);
            ounscale = __builtin_ldexpf(1.0f, -15 - sv);
        }
    }
    // keys by threads 0-255 and values by 256-511 (NT = 2), or both by every thread
    auto unpack = [&](PfLds& Ld, const PfRawL<BIG>& Rr, int nt) __attribute__((always_inline)) {
        if constexpr (NT == 1) pf_unpack<KK, KV, RING, BIG, 0>(Ld, Rr, a, nt, quant, tid, vmul);
        else if (tid < 256) pf_unpack<KK, KV, RING, BIG, 1>(Ld, Rr, a, nt, quant, tid, vmul);
        else pf_unpack<KK, KV, RING, BIG, 2>(Ld, Rr, a, nt, quant, tid - 256, vmul);
    };
    if (nb > 0) unpack(L[0], RW[0], nt_of(0));
    // iteration i: L[i & 1] holds block i, RW[(i + 1) & 1] raw block i + 1 (loaded during
    // block i - 1); RW[i & 1] is free for block i + 2
    auto step = [&](int i, PfLds& Lc, PfLds& Ln, PfRawL<BIG>& Rn, PfRawL<BIG>& Rf) __attribute__((always_inline)) {
        pf_wait_vm0();
        __syncthreads();
        if (i + 1 < nb) unpack(Ln, Rn, nt_of(i + 1));
        if (i + 2 < nb) pf_dma<KK, KV, RING, BIG, 4 * NT>(Rf, a, SK, SV, tb_of(i + 2), nt_of(i + 2), wave, lane);
        compute(Lc, tb_of(i), nt_of(i));
    };
    for (int i = 0; i < nb; i += 2) {
        step(i, L[0], L[1], RW[1], RW[0]);
        if (i + 1 < nb) step(i + 1, L[1], L[0], RW[0], RW[1]);
    }
    pf_wait_vm0();
    // ---- partial result of the split: m, l and acc[128] per query (dims 32 b + i(r)) --------
    if (tile >= a.tiles) return;                                    // the odd tile group's empty half
    float* pp = a.partials + (((((int64_t)head * a.tiles + tile) * S + sp) * kG + h) * kPfQ + j) * (kD + 2);
    if (hh == 0) {
        pp[0] = mrun;
        pp[1] = lrun;
    }
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) pp[2 + 32 * b + 8 * (r >> 2) + 4 * hh + (r & 3)] = O[b][r] * ounscale;
}

// One workgroup of 128 threads per (query, query head): merge the splits; the quantized
// splits' value sum is rotated back for KVarN values.
template <bool KVARN_V>
__global__ __launch_bounds__(128) void k_prefill_merge(PrefillArgs a)
{
    __shared__ float vq[kD];
    __shared__ float ML[2];
    const int d = threadIdx.x;
    const int qi = blockIdx.x / a.g.n_q_heads, qh = blockIdx.x % a.g.n_q_heads;
    const int head = qh / kG, h = qh % kG, tile = qi / kPfQ, j = qi % kPfQ;
    const int S = a.splits_q + a.splits_t;
    const float* base = a.partials + ((((int64_t)head * a.tiles + tile) * S) * kG + h) * kPfQ * (kD + 2) + (int64_t)j * (kD + 2);
    const int64_t sstride = (int64_t)kG * kPfQ * (kD + 2);
    float M = kNeg;
    for (int s = 0; s < S; ++s) M = fmaxf(M, base[s * sstride]);
    float L = 0.0f, aq = 0.0f, at = 0.0f;
    for (int s = 0; s < S; ++s) {
        const float* p = base + s * sstride;
        const float w = p[1] > 0.0f ? __builtin_amdgcn_exp2f(p[0] - M) : 0.0f;
        L = fmaf(p[1], w, L);
        if (s < a.splits_q) aq = fmaf(p[2 + d], w, aq);
        else at = fmaf(p[2 + d], w, at);
    }
    vq[d] = aq;
    if (KVARN_V) {
        for (int span = 1; span < kD; span <<= 1) {
            __syncthreads();
            if (d < kD / 2) {
                const int lo = d & (span - 1);
                const int i = ((d - lo) << 1) | lo;
                const float x = vq[i], y = vq[i + span];
                vq[i] = x + y;
                vq[i + span] = x - y;
            }
        }
    }
    __syncthreads();
    if (d == 0) ML[1] = L;
    __syncthreads();
    const float q = KVARN_V ? vq[d] * (1.0f / 128.0f) : vq[d];
    a.out[((int64_t)qi * a.g.n_q_heads + qh) * kD + d] = (q + at) / ML[1];
}

template <int KK, int KV>
int launch_pf(const PrefillArgs& a, hipStream_t st)
{
    // quantized splits and ring splits: one kernel each (their staging differs)
    constexpr int NQ = 2;                            // tiles per workgroup
    if (a.splits_q > 0)
        hipLaunchKernelGGL((k_prefill<KK, KV, false>), dim3(a.g.n_kv_heads * ((a.tiles + NQ - 1) / NQ) * a.splits_q),
                           dim3(256 * NQ), 0, st, a);
    if (a.splits_t > 0)
        hipLaunchKernelGGL((k_prefill<KK, KV, true>), dim3(a.g.n_kv_heads * ((a.tiles + 1) / 2) * a.splits_t),
                           dim3(512), 0, st, a);
    return (int)hipGetLastError();
}

template <int KK>
int launch_pf_v(const PrefillArgs& a, hipStream_t st)
{
    switch (fkind(a.g.fmt_v)) {
    case KIND_BF16: return launch_pf<KK, KIND_BF16>(a, st);
    case KIND_Q0: return launch_pf<KK, KIND_Q0>(a, st);
    case KIND_Q1: return launch_pf<KK, KIND_Q1>(a, st);
    case KIND_KVARN: return launch_pf<KK, KIND_KVARN>(a, st);
    default: return launch_pf<KK, KIND_KVARN1>(a, st);
    }
}

}  // namespace

int launch_prefill(const PrefillArgs& a, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    int rc;
    switch (fkind(a.g.fmt_k)) {
    case KIND_BF16: rc = launch_pf_v<KIND_BF16>(a, st); break;
    case KIND_Q0: rc = launch_pf_v<KIND_Q0>(a, st); break;
    case KIND_Q1: rc = launch_pf_v<KIND_Q1>(a, st); break;
    case KIND_KVARN: rc = launch_pf_v<KIND_KVARN>(a, st); break;
    default: rc = launch_pf_v<KIND_KVARN1>(a, st); break;
    }
    if (rc) return rc;
    const int n = a.n_new * a.g.n_q_heads;
    if (kind_paged(fkind(a.g.fmt_v)))
        hipLaunchKernelGGL(k_prefill_merge<true>, dim3(n), dim3(128), 0, st, a);
    else
        hipLaunchKernelGGL(k_prefill_merge<false>, dim3(n), dim3(128), 0, st, a);
    return (int)hipGetLastError();
}

}  // namespace kvq
