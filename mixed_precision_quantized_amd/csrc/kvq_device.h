// kvq_device.h -- device helpers shared by the gfx950 kernels: format traits, bit-exact
// conversions and packed-code access.
//
// Numeric rules every encode kernel follows (the cache's definition): binary32 with each
// operation rounded to nearest-even, no contraction of a*b+c into an FMA (the encode
// translation units are built with -ffp-contract=off and say so with a pragma),
// subnormals kept, '/' and sqrtf correctly rounded.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

// The split that workgroup b of a decode launch runs: every quantized split first
// (sequence by sequence, then head by head), every ring split after them, so that in a
// launch of several waves the small ring splits fill the end.  Its partial goes to slot
// wg_base + head (splits_q + splits_t) + sp of the sequence, sp counting the quantized
// splits first.
struct DecodeWork { int e, head, sp, slot; };
__device__ inline DecodeWork decode_work(const DecodeArgs& a, int b)
{
    const bool quant = b < a.q_wgs;
    const int r0 = quant ? b : b - a.q_wgs;
    int e = 0;
    for (int i = 1; i < a.n_seqs; ++i)
        if ((quant ? a.seqs[i].q_base : a.seqs[i].t_base) <= r0) e = i;
    const DecodeSeq& s = a.seqs[e];
    const int rr = r0 - (quant ? s.q_base : s.t_base);
    const int ns = quant ? s.splits_q : s.splits_t;
    DecodeWork w;
    w.e = e;
    w.head = rr / ns;
    w.sp = (quant ? 0 : s.splits_q) + rr % ns;
    w.slot = s.wg_base + w.head * (s.splits_q + s.splits_t) + w.sp;
    return w;
}

// ------------------------------------------------------------------ format traits
// Bits N per code of each format (bf16 = 16).
__host__ __device__ constexpr int fbits(int f)
{
    return f == 0 ? 16 : f == 1 ? 2 : f == 2 ? 2 : f == 3 ? 3 : f == 4 ? 3 : f == 5 ? 4 : f == 6 ? 4
         : f == 7 ? 5 : f == 8 ? 5 : f == 9 ? 6 : f == 10 ? 6 : f == 11 ? 8 : f == 12 ? 8
         : f == 13 ? 2 : f == 14 ? 3 : f == 15 ? 4 : f == 16 ? 5 : f == 17 ? 6 : f == 18 ? 8
         : f == 19 ? 2 : f == 20 ? 3 : f == 21 ? 4 : f == 22 ? 5 : f == 23 ? 6 : f == 24 ? 8 : 0;
}
__host__ __device__ constexpr int fkind(int f)
{
    return f == 0 ? KIND_BF16 : f >= 19 ? KIND_KVARN1 : f >= 13 ? KIND_KVARN
         : ((f - 1) % 2 == 0 ? KIND_Q0 : KIND_Q1);
}
__host__ __device__ constexpr int fcode_bytes(int f) { return f == 0 ? 256 : 16 * fbits(f); }
__host__ __device__ constexpr int fscale_halves(int f)
{
    return fkind(f) == KIND_BF16 ? 0 : (kind_affine(fkind(f)) ? 8 : 4);
}

// ------------------------------------------------------------------ conversions
// bf16(x): round to nearest even on the upper half (finite inputs).
__device__ __forceinline__ uint16_t bf16_rne(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp16s(x): round to nearest even to binary16 with integer operations (independent of
// the denormal mode), saturate to +-65504, a zero result is +0.
__device__ __forceinline__ uint16_t fp16s_rne(float x)
{
    uint32_t u = __float_as_uint(x);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t a = u & 0x7FFFFFFFu;
    uint32_t r;
    if (a >= 0x477FF000u) {                 // |x| >= 65520: the nearest-even result is inf
        r = 0x7BFFu;
    } else if (a >= 0x38800000u) {          // |x| >= 2^-14: normal binary16
        uint32_t h = ((a >> 23) - 112u) << 10 | ((a & 0x7FFFFFu) >> 13);
        uint32_t rem = a & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;
        r = h;
    } else {                                // subnormal binary16 or zero, quantum 2^-24
        uint32_t e = a >> 23;
        if (e < 102u) {
            r = 0;
        } else {
            uint32_t m = (a & 0x7FFFFFu) | 0x800000u;
            uint32_t sh = 126u - e;          // 14..24
            uint32_t q = m >> sh;
            uint32_t rem = m & ((1u << sh) - 1u);
            uint32_t half = 1u << (sh - 1u);
            if (rem > half || (rem == half && (q & 1u))) q += 1u;
            r = q;
        }
    }
    return r ? (uint16_t)(r | sign) : (uint16_t)0;
}

__device__ __forceinline__ float fp16_to_f32(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// A canonical 16-bit value (ring rows): bf16, or binary16 for an F16 tail.
__device__ __forceinline__ float canon_to_f32(uint32_t h, bool f16)
{
    return f16 ? fp16_to_f32(h & 0xFFFFu) : bf16_to_f32(h & 0xFFFFu);
}
// The canonical 16 bits of an input value: bf16 by RNE, or binary16 by RNE, saturated to
// +-65504 with zero as +0 (the same conversion as the block scales).
__device__ __forceinline__ uint32_t canon_bits(float x, bool f16)
{
    return f16 ? (uint32_t)fp16s_rne(x) : (uint32_t)bf16_rne(x);
}

// ------------------------------------------------------------------ packed codes
// Extract code i (0-based within a group) of N bits from a little-endian bit stream held
// in 32-bit words w[] (word 0 holds stream bits 0..31).
template <int N, int NW>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[NW], int i)
{
    const int bit = i * N;
    const int wi = bit >> 5;
    const int sh = bit & 31;
    uint32_t v = w[wi] >> sh;
    if (sh + N > 32) v |= w[wi + 1] << (32 - sh);
    return v & ((1u << N) - 1u);
}

}  // namespace kvq
