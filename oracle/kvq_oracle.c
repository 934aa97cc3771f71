/*
 * kvq_oracle.c -- plain CPU oracle; see kvq_oracle.h for the scope, the sources
 * ([P1]..[P5]) and the numeric ground rules.
 *
 * TEST INFRASTRUCTURE ONLY: never linked into, loaded by or called from the product.
 *
 * Written for readability, not speed: every step follows the definition in the order
 * it is stated, one scalar at a time.  Build: -std=c11 -O2 -ffp-contract=off
 * -fno-fast-math (x86-64 SSE2, IEEE binary32 with round-to-nearest-even).
 */
#include "kvq_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ======================================================================== */
/* Scalar conversions                                                        */
/* ======================================================================== */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float f32_from_bits(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

float kvo_f32_from_bf16(uint16_t b)
{
    /* bf16 is by definition the upper half of a binary32 pattern. */
    return f32_from_bits((uint32_t)b << 16);
}

/* The canonical 16-bit type of the cache's values: bf16 (default) or binary16 (an F16
 * tail, "Экспериментальные методы квантизации KV-кэша в BeeLLama.cpp v0.4.0", section
 * "KV Cache Precision Tail": the tail is BF16 or F16).  Every function below that takes
 * canonical 16-bit values reads them in this type. */
static int g_canon_f16 = 0;
void kvo_set_canonical_f16(int on) { g_canon_f16 = on ? 1 : 0; }
int kvo_canonical_f16(void) { return g_canon_f16; }
static double f64_from_canon(uint16_t b);

/* Round x (finite) to the nearest multiple of 'quantum' (a power of two), ties to an
 * even multiple.  x/quantum is exact in binary64 because x has at most 24 significant
 * bits; rint() in the default rounding mode is round-half-to-even. */
static double round_to_quantum_even(double x, double quantum)
{
    double r = x / quantum;
    return rint(r) * quantum;
}

uint16_t kvo_bf16_from_f32(float xf)
{
    /* Nearest value with an 8-bit significand (7 stored bits), exponent range of
     * binary32; ties to even.  Quantum for |x| in [2^e, 2^(e+1)) is 2^(e-7); for
     * subnormal binary32 inputs the quantum is the binary32 subnormal spacing scaled
     * to 8 significant bits of the top-half pattern, i.e. 2^-133. */
    double x = (double)xf;
    if (x == 0.0) return (uint16_t)(f32_bits(xf) >> 16);   /* keeps the sign of zero */
    double ax = fabs(x);
    double quantum;
    if (ax < ldexp(1.0, -126)) {
        quantum = ldexp(1.0, -133);
    } else {
        int e;
        frexp(ax, &e);          /* ax = f * 2^e, f in [0.5, 1) -> ax in [2^(e-1), 2^e) */
        quantum = ldexp(1.0, (e - 1) - 7);
    }
    double r = round_to_quantum_even(x, quantum);
    /* r is a binary32 value whose low 16 bits are zero (or it overflowed to 2^128). */
    if (fabs(r) >= ldexp(1.0, 128)) {
        return (uint16_t)(x < 0 ? 0xFF80u : 0x7F80u);       /* +-inf */
    }
    float rf = (float)r;                                    /* exact */
    uint32_t u = f32_bits(rf);
    return (uint16_t)(u >> 16);
}

double kvo_f64_from_fp16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);                          /* subnormal: m * 2^-24 */
    } else if (e == 31) {
        v = m ? NAN : INFINITY;
    } else {
        v = ldexp(1.0 + (double)m / 1024.0, e - 15);
    }
    return sign ? -v : v;
}

/* Encode an exactly representable binary16 value (|v| <= 65504) as bits. */
static uint16_t fp16_bits_of_exact(double v)
{
    uint16_t sign = (v < 0) ? 0x8000u : 0;
    double a = fabs(v);
    if (a == 0.0) return 0;                                 /* zero -> +0 */
    if (a < ldexp(1.0, -14)) {                              /* subnormal */
        double m = a / ldexp(1.0, -24);
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e;
    double f = frexp(a, &e);                                /* a = f*2^e, f in [0.5,1) */
    int E = e - 1;                                          /* a in [2^E, 2^(E+1)) */
    double mant = (a / ldexp(1.0, E) - 1.0) * 1024.0;       /* exact integer 0..1023 */
    (void)f;
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)mant);
}

uint16_t kvo_fp16s_from_f32(float xf)
{
    double x = (double)xf;
    if (x == 0.0) return 0;
    double ax = fabs(x);
    double quantum;
    if (ax < ldexp(1.0, -14)) {
        quantum = ldexp(1.0, -24);                          /* binary16 subnormal spacing */
    } else {
        int e;
        frexp(ax, &e);
        quantum = ldexp(1.0, (e - 1) - 10);                 /* 11-bit significand */
    }
    double r = round_to_quantum_even(x, quantum);
    /* Saturation: anything at or beyond the largest finite binary16 becomes +-65504.
     * (Every finite x with |x| >= 65504 rounds either to 65504 or to infinity.) */
    if (r >= 65504.0) r = 65504.0;
    if (r <= -65504.0) r = -65504.0;
    if (r == 0.0) return 0;                                 /* zero result -> +0 */
    return fp16_bits_of_exact(r);
}

static float f32_from_fp16(uint16_t h) { return (float)kvo_f64_from_fp16(h); }
static double f64_from_canon(uint16_t b) { return g_canon_f16 ? kvo_f64_from_fp16(b) : (double)kvo_f32_from_bf16(b); }
static float f32_from_canon(uint16_t b) { return (float)f64_from_canon(b); }

/* ======================================================================== */
/* Format table                                                              */
/* ======================================================================== */

int kvo_format_info(int fmt, int* bits, int* kind, int* code_bytes, int* scale_bytes,
                    int* page_bytes)
{
    int N, K;
    switch (fmt) {
    case KVO_BF16:   N = 16; K = KVO_KIND_BF16; break;
    case KVO_Q2_0:   N = 2; K = KVO_KIND_Q0; break;
    case KVO_Q2_1:   N = 2; K = KVO_KIND_Q1; break;
    case KVO_Q3_0:   N = 3; K = KVO_KIND_Q0; break;
    case KVO_Q3_1:   N = 3; K = KVO_KIND_Q1; break;
    case KVO_Q4_0:   N = 4; K = KVO_KIND_Q0; break;
    case KVO_Q4_1:   N = 4; K = KVO_KIND_Q1; break;
    case KVO_Q5_0:   N = 5; K = KVO_KIND_Q0; break;
    case KVO_Q5_1:   N = 5; K = KVO_KIND_Q1; break;
    case KVO_Q6_0:   N = 6; K = KVO_KIND_Q0; break;
    case KVO_Q6_1:   N = 6; K = KVO_KIND_Q1; break;
    case KVO_Q8_0:   N = 8; K = KVO_KIND_Q0; break;
    case KVO_Q8_1:   N = 8; K = KVO_KIND_Q1; break;
    case KVO_KVARN2: N = 2; K = KVO_KIND_KVARN; break;
    case KVO_KVARN3: N = 3; K = KVO_KIND_KVARN; break;
    case KVO_KVARN4: N = 4; K = KVO_KIND_KVARN; break;
    case KVO_KVARN5: N = 5; K = KVO_KIND_KVARN; break;
    case KVO_KVARN6: N = 6; K = KVO_KIND_KVARN; break;
    case KVO_KVARN8: N = 8; K = KVO_KIND_KVARN; break;
    case KVO_KVARN2_1: N = 2; K = KVO_KIND_KVARN1; break;
    case KVO_KVARN3_1: N = 3; K = KVO_KIND_KVARN1; break;
    case KVO_KVARN4_1: N = 4; K = KVO_KIND_KVARN1; break;
    case KVO_KVARN5_1: N = 5; K = KVO_KIND_KVARN1; break;
    case KVO_KVARN6_1: N = 6; K = KVO_KIND_KVARN1; break;
    case KVO_KVARN8_1: N = 8; K = KVO_KIND_KVARN1; break;
    default: return -1;
    }
    if (bits) *bits = N;
    if (kind) *kind = K;
    if (code_bytes) *code_bytes = (K == KVO_KIND_BF16) ? 256 : 16 * N;
    if (scale_bytes) *scale_bytes = (K == KVO_KIND_BF16) ? 0 : ((K == KVO_KIND_Q1 || K == KVO_KIND_KVARN1) ? 16 : 8);
    if (page_bytes) *page_bytes = (K == KVO_KIND_KVARN || K == KVO_KIND_KVARN1) ? 256 : 0;
    return 0;
}

/* ======================================================================== */
/* Block encoders                                                            */
/* ======================================================================== */

/* clamp(rint(t) + off, 0, top) with rint = round-half-even in binary32. */
static uint8_t code_from_t(float t, int off, int top)
{
    float r = rintf(t);
    float v = r + (float)off;
    if (v < 0.0f) v = 0.0f;
    if (v > (float)top) v = (float)top;
    return (uint8_t)v;
}

void kvo_encode_block_q0(int N, const float x[32], uint16_t* d16, uint8_t u[32])
{
    const int off = 1 << (N - 1);
    const int top = (1 << N) - 1;
    /* 1. max and min of the block */
    float mx = x[0], mn = x[0];
    for (int i = 1; i < 32; ++i) {
        if (x[i] > mx) mx = x[i];
        if (x[i] < mn) mn = x[i];
    }
    /* 2. signed max-magnitude element; a tie |mx| == |mn| goes to the positive one */
    float m = (mx >= -mn) ? mx : mn;
    /* 3. d = m / -2^(N-1), stored as saturating fp16 */
    float q = m / -(float)off;
    uint16_t d = kvo_fp16s_from_f32(q);
    *d16 = d;
    /* 4. zero scale: every code is the offset (the value 0) */
    if (d == 0) {
        for (int i = 0; i < 32; ++i) u[i] = (uint8_t)off;
        return;
    }
    /* 5. reciprocal once, then multiply and round half to even */
    float df = f32_from_fp16(d);
    float inv = 1.0f / df;
    for (int i = 0; i < 32; ++i) {
        float t = x[i] * inv;
        u[i] = code_from_t(t, off, top);
    }
}

void kvo_encode_block_q1(int N, const float x[32], uint16_t* d16, uint16_t* m16, uint8_t u[32])
{
    const int top = (1 << N) - 1;
    float mx = x[0], mn = x[0];
    for (int i = 1; i < 32; ++i) {
        if (x[i] > mx) mx = x[i];
        if (x[i] < mn) mn = x[i];
    }
    float dr = mx - mn;
    float dq = dr / (float)top;
    uint16_t d = kvo_fp16s_from_f32(dq);
    uint16_t m = kvo_fp16s_from_f32(mn);
    *d16 = d;
    *m16 = m;
    if (d == 0) {
        for (int i = 0; i < 32; ++i) u[i] = 0;
        return;
    }
    float df = f32_from_fp16(d);
    float mf = f32_from_fp16(m);
    float inv = 1.0f / df;
    for (int i = 0; i < 32; ++i) {
        float diff = x[i] - mf;
        float t = diff * inv;
        u[i] = code_from_t(t, 0, top);
    }
}

void kvo_pack_codes(int N, const uint8_t u[128], uint8_t* out)
{
    memset(out, 0, (size_t)(16 * N));
    for (int j = 0; j < 128; ++j) {
        for (int k = 0; k < N; ++k) {
            int bit = (u[j] >> k) & 1;
            int s = j * N + k;
            out[s / 8] |= (uint8_t)(bit << (s % 8));
        }
    }
}

void kvo_unpack_codes(int N, const uint8_t* in, uint8_t u[128])
{
    for (int j = 0; j < 128; ++j) {
        int v = 0;
        for (int k = 0; k < N; ++k) {
            int s = j * N + k;
            v |= ((in[s / 8] >> (s % 8)) & 1) << k;
        }
        u[j] = (uint8_t)v;
    }
}

/* ======================================================================== */
/* KVarN: rotation, Sinkhorn balancing, page encoder                         */
/* ======================================================================== */

void kvo_fwht128_f32(float y[128])
{
    for (int h = 1; h < 128; h <<= 1) {
        for (int i = 0; i < 128; ++i) {
            if (i & h) continue;
            float a = y[i], b = y[i + h];
            y[i] = a + b;
            y[i + h] = a - b;
        }
    }
}

/* tree128(v): for w = 64, 32, ..., 1: v[i] += v[i+w] for i < w; result v[0]. */
static float tree128(float v[128])
{
    for (int w = 64; w >= 1; w >>= 1)
        for (int i = 0; i < w; ++i) v[i] = v[i] + v[i + w];
    return v[0];
}

static float guard_scale(float s)
{
    /* A zero, subnormal or NaN mean square would make a later reciprocal blow up:
     * replace it by 1 (READING: guard of the Sinkhorn iteration). */
    if (!(s >= FLT_MIN)) return 1.0f;
    return s;
}

void kvo_sinkhorn128(const float* A, int iters, float r2[128], float c2[128])
{
    float v[128], ic[128], ir[128];
    const float inv128 = 1.0f / 128.0f;
    for (int j = 0; j < 128; ++j) c2[j] = 1.0f;
    for (int t = 0; t < 128; ++t) r2[t] = 1.0f;
    for (int it = 0; it < iters; ++it) {
        /* row step: mean over channels of A / c2, per token */
        for (int j = 0; j < 128; ++j) ic[j] = 1.0f / c2[j];
        for (int t = 0; t < 128; ++t) {
            for (int j = 0; j < 128; ++j) v[j] = A[t * 128 + j] * ic[j];
            r2[t] = guard_scale(tree128(v) * inv128);
        }
        /* column step: mean over tokens of A / r2, per channel */
        for (int t = 0; t < 128; ++t) ir[t] = 1.0f / r2[t];
        for (int j = 0; j < 128; ++j) {
            for (int t = 0; t < 128; ++t) v[t] = A[t * 128 + j] * ir[t];
            c2[j] = guard_scale(tree128(v) * inv128);
        }
    }
}

#define KVARN_ITERS 8

static void encode_page_kvarn_impl(int N, int affine, const uint16_t* X, uint8_t* codes,
                                   uint16_t* scales, uint16_t* cscale);

void kvo_encode_page_kvarn(int N, const uint16_t* X, uint8_t* codes, uint16_t* scales,
                           uint16_t* cscale)
{
    encode_page_kvarn_impl(N, 0, X, codes, scales, cscale);
}

void kvo_encode_page_kvarn_q1(int N, const uint16_t* X, uint8_t* codes, uint16_t* scales,
                              uint16_t* cscale)
{
    encode_page_kvarn_impl(N, 1, X, codes, scales, cscale);
}

static void encode_page_kvarn_impl(int N, int affine, const uint16_t* X, uint8_t* codes,
                                   uint16_t* scales, uint16_t* cscale)
{
    float* Y = (float*)malloc(sizeof(float) * 128 * 128);
    float* A = (float*)malloc(sizeof(float) * 128 * 128);
    float r2[128], c2[128], ic16[128];
    /* 1. rotation of every token vector */
    for (int t = 0; t < 128; ++t) {
        float* y = Y + t * 128;
        for (int i = 0; i < 128; ++i) y[i] = f32_from_canon(X[t * 128 + i]);
        kvo_fwht128_f32(y);
    }
    /* 2. squares */
    for (int k = 0; k < 128 * 128; ++k) A[k] = Y[k] * Y[k];
    /* 3. Sinkhorn on squared scales */
    kvo_sinkhorn128(A, KVARN_ITERS, r2, c2);
    /* 4. channel scales: fp16 of the root mean square; a zero becomes 1.0 */
    for (int j = 0; j < 128; ++j) {
        uint16_t c = kvo_fp16s_from_f32(sqrtf(c2[j]));
        if (c == 0) c = 0x3C00u;
        cscale[j] = c;
        ic16[j] = 1.0f / f32_from_fp16(c);
    }
    /* 5./6. normalize each channel, then block quantization (symmetric, or affine for
     * an _1 base) and packing */
    const int cb = 16 * N;
    for (int t = 0; t < 128; ++t) {
        float w[128];
        uint8_t u[128];
        for (int j = 0; j < 128; ++j) w[j] = Y[t * 128 + j] * ic16[j];
        for (int b = 0; b < 4; ++b) {
            if (affine)
                kvo_encode_block_q1(N, w + 32 * b, &scales[t * 8 + 2 * b], &scales[t * 8 + 2 * b + 1], u + 32 * b);
            else
                kvo_encode_block_q0(N, w + 32 * b, &scales[t * 4 + b], u + 32 * b);
        }
        kvo_pack_codes(N, u, codes + (size_t)t * cb);
    }
    free(Y);
    free(A);
}

/* ======================================================================== */
/* Token and stream encoders                                                 */
/* ======================================================================== */

int kvo_encode_token(int fmt, const uint16_t* x, uint8_t* codes, uint16_t* scales)
{
    int N, kind, cb, sb, pb;
    if (kvo_format_info(fmt, &N, &kind, &cb, &sb, &pb) != 0) return -1;
    if (kind == KVO_KIND_BF16) {
        memcpy(codes, x, 256);                  /* identity: the bf16 row itself */
        return 0;
    }
    if (kind == KVO_KIND_KVARN || kind == KVO_KIND_KVARN1) return -1;      /* pages only */
    float xf[128];
    uint8_t u[128];
    for (int i = 0; i < 128; ++i) xf[i] = f32_from_canon(x[i]);
    for (int b = 0; b < 4; ++b) {
        if (kind == KVO_KIND_Q0) {
            kvo_encode_block_q0(N, xf + 32 * b, &scales[b], u + 32 * b);
        } else {
            kvo_encode_block_q1(N, xf + 32 * b, &scales[2 * b], &scales[2 * b + 1], u + 32 * b);
        }
    }
    kvo_pack_codes(N, u, codes);
    return 0;
}

int kvo_encode_stream(int fmt, int64_t n_q, const uint16_t* x, uint8_t* codes,
                      uint16_t* scales, uint16_t* cscale)
{
    int N, kind, cb, sb, pb;
    if (kvo_format_info(fmt, &N, &kind, &cb, &sb, &pb) != 0 || n_q < 0) return -1;
    if (kind == KVO_KIND_KVARN || kind == KVO_KIND_KVARN1) {
        if (n_q % KVO_PAGE) return -1;
        for (int64_t p = 0; p < n_q / KVO_PAGE; ++p) {
            encode_page_kvarn_impl(N, kind == KVO_KIND_KVARN1, x + p * 128 * 128, codes + p * 128 * cb,
                                   scales + p * 128 * (sb / 2), cscale + p * 128);
        }
        return 0;
    }
    for (int64_t t = 0; t < n_q; ++t) {
        kvo_encode_token(fmt, x + t * 128, codes + t * cb, scales ? scales + t * (sb / 2) : NULL);
    }
    return 0;
}

/* ======================================================================== */
/* Decode side (binary64)                                                    */
/* ======================================================================== */

static int popcount_u32(unsigned v) { int c = 0; while (v) { c += v & 1u; v >>= 1; } return c; }

int kvo_dequant_token(int fmt, const uint8_t* codes, const uint16_t* scales,
                      const uint16_t* cscale_row, double out[128])
{
    int N, kind, cb, sb, pb;
    if (kvo_format_info(fmt, &N, &kind, &cb, &sb, &pb) != 0) return -1;
    if (kind == KVO_KIND_BF16) {
        for (int i = 0; i < 128; ++i) {
            uint16_t b = (uint16_t)(codes[2 * i] | (codes[2 * i + 1] << 8));
            out[i] = (double)kvo_f32_from_bf16(b);
        }
        return 0;
    }
    uint8_t u[128];
    kvo_unpack_codes(N, codes, u);
    const int off = 1 << (N - 1);
    if (kind == KVO_KIND_Q0) {
        for (int j = 0; j < 128; ++j)
            out[j] = (double)(u[j] - off) * kvo_f64_from_fp16(scales[j / 32]);
        return 0;
    }
    if (kind == KVO_KIND_Q1) {
        for (int j = 0; j < 128; ++j) {
            double d = kvo_f64_from_fp16(scales[2 * (j / 32)]);
            double m = kvo_f64_from_fp16(scales[2 * (j / 32) + 1]);
            out[j] = m + (double)u[j] * d;
        }
        return 0;
    }
    /* kvarn: Yhat = c * (the block-quantized value) in the rotated domain, then
     * x = H Yhat / 128 */
    double yh[128];
    for (int j = 0; j < 128; ++j) {
        const double w = kind == KVO_KIND_KVARN1
            ? kvo_f64_from_fp16(scales[2 * (j / 32) + 1]) + (double)u[j] * kvo_f64_from_fp16(scales[2 * (j / 32)])
            : kvo_f64_from_fp16(scales[j / 32]) * (double)(u[j] - off);
        yh[j] = kvo_f64_from_fp16(cscale_row[j]) * w;
    }
    for (int i = 0; i < 128; ++i) {
        double s = 0.0;
        for (int j = 0; j < 128; ++j) {
            double h = (popcount_u32((unsigned)(i & j)) & 1) ? -1.0 : 1.0;
            s += h * yh[j];
        }
        out[i] = s / 128.0;
    }
    return 0;
}

int kvo_dequant_stream(int fmt, int64_t n_q, const uint8_t* codes, const uint16_t* scales,
                       const uint16_t* cscale, double* out)
{
    int N, kind, cb, sb, pb;
    if (kvo_format_info(fmt, &N, &kind, &cb, &sb, &pb) != 0 || n_q < 0) return -1;
    for (int64_t t = 0; t < n_q; ++t) {
        const uint16_t* crow = (kind == KVO_KIND_KVARN || kind == KVO_KIND_KVARN1) ? cscale + (t / KVO_PAGE) * 128 : NULL;
        kvo_dequant_token(fmt, codes + t * cb, scales ? scales + t * (sb / 2) : NULL, crow,
                          out + t * 128);
    }
    return 0;
}

/* ======================================================================== */
/* Precision tail state machine                                              */
/* ======================================================================== */

int64_t kvo_granule(int fmt_k, int fmt_v)
{
    int kk = -1, kv = -1;
    kvo_format_info(fmt_k, NULL, &kk, NULL, NULL, NULL);
    kvo_format_info(fmt_v, NULL, &kv, NULL, NULL, NULL);
    return (kk == KVO_KIND_KVARN || kv == KVO_KIND_KVARN || kk == KVO_KIND_KVARN1 || kv == KVO_KIND_KVARN1)
               ? KVO_PAGE : 1;
}

int64_t kvo_ring_capacity(int64_t T, int64_t G)
{
    if (T < 0 || G < 1) return -1;
    int64_t need = T + G - 1;                     /* largest possible ring occupancy */
    return G * ((need + G - 1) / G);
}

int64_t kvo_nq_after(int64_t n_q, int64_t n, int64_t keep, int64_t G)
{
    int64_t over = n - keep;
    if (over < 0) over = 0;
    int64_t cand = G * (over / G);
    return cand > n_q ? cand : n_q;
}

int kvo_ring_image(int64_t n, int64_t n_q, int64_t R, const uint16_t* x, uint16_t* ring)
{
    if (n < n_q || n_q < 0) return -1;
    if (n > n_q && R <= 0) return -1;
    if (n - n_q > R) return -1;
    for (int64_t p = n_q; p < n; ++p)
        memcpy(ring + (p % R) * 128, x + p * 128, 256);
    return 0;
}

/* ======================================================================== */
/* Attention reference                                                       */
/* ======================================================================== */

int kvo_attention(int64_t n, int64_t n_q, int fmt_k, int fmt_v,
                  const uint8_t* kq_codes, const uint16_t* kq_scales, const uint16_t* kq_cscale,
                  const uint8_t* vq_codes, const uint16_t* vq_scales, const uint16_t* vq_cscale,
                  const uint16_t* k_tail, const uint16_t* v_tail,
                  int g, const double* q, double sigma, double* out)
{
    int Nk, kk, cbk, sbk, pbk, Nv, kv, cbv, sbv, pbv;
    if (kvo_format_info(fmt_k, &Nk, &kk, &cbk, &sbk, &pbk) != 0) return -1;
    if (kvo_format_info(fmt_v, &Nv, &kv, &cbv, &sbv, &pbv) != 0) return -1;
    if (n == 0) return -4;
    if (n < 0 || n_q < 0 || n_q > n || g <= 0) return -1;
    /* dequantize every token once (K and V), then one softmax per query head */
    double* K = (double*)malloc(sizeof(double) * (size_t)n * 128);
    double* V = (double*)malloc(sizeof(double) * (size_t)n * 128);
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    if (!K || !V || !s) { free(K); free(V); free(s); return -1; }
    kvo_dequant_stream(fmt_k, n_q, kq_codes, kq_scales, kq_cscale, K);
    kvo_dequant_stream(fmt_v, n_q, vq_codes, vq_scales, vq_cscale, V);
    for (int64_t t = n_q; t < n; ++t) {
        for (int i = 0; i < 128; ++i) {
            K[t * 128 + i] = f64_from_canon(k_tail[(t - n_q) * 128 + i]);
            V[t * 128 + i] = f64_from_canon(v_tail[(t - n_q) * 128 + i]);
        }
    }
    for (int h = 0; h < g; ++h) {
        const double* qh = q + h * 128;
        double M = -INFINITY;
        for (int64_t t = 0; t < n; ++t) {
            double acc = 0.0;
            for (int i = 0; i < 128; ++i) acc += qh[i] * K[t * 128 + i];
            s[t] = sigma * acc;
            if (s[t] > M) M = s[t];
        }
        double l = 0.0;
        double o[128];
        for (int i = 0; i < 128; ++i) o[i] = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            double p = exp(s[t] - M);
            l += p;
            for (int i = 0; i < 128; ++i) o[i] += p * V[t * 128 + i];
        }
        for (int i = 0; i < 128; ++i) out[h * 128 + i] = o[i] / l;
    }
    free(K);
    free(V);
    free(s);
    return 0;
}

/* ======================================================================== */
/* Attention fidelity (KL divergence of attention distributions)           */
/* ======================================================================== */

int kvo_attention_kld(int64_t n, int64_t n_q, int fmt_k, const uint8_t* kq_codes,
                      const uint16_t* kq_scales, const uint16_t* kq_cscale,
                      const uint16_t* k_exact, int g, const double* q, double sigma, double* kld)
{
    int N, kind, cb, sb, pb;
    if (kvo_format_info(fmt_k, &N, &kind, &cb, &sb, &pb) != 0) return -1;
    if (n == 0) return -4;
    if (n < 0 || n_q < 0 || n_q > n || g <= 0 || !k_exact || !q || !kld) return -1;
    double* K = (double*)malloc(sizeof(double) * (size_t)n * 128);
    double* se = (double*)malloc(sizeof(double) * (size_t)n);
    double* sq = (double*)malloc(sizeof(double) * (size_t)n);
    if (!K || !se || !sq) { free(K); free(se); free(sq); return -1; }
    /* the cache's keys: dequantized below n_q, the exact bf16 rows above */
    if (n_q > 0) kvo_dequant_stream(fmt_k, n_q, kq_codes, kq_scales, kq_cscale, K);
    for (int64_t t = n_q; t < n; ++t)
        for (int i = 0; i < 128; ++i) K[t * 128 + i] = f64_from_canon(k_exact[t * 128 + i]);
    for (int h = 0; h < g; ++h) {
        const double* qh = q + h * 128;
        double Me = -INFINITY, Mq = -INFINITY;
        for (int64_t t = 0; t < n; ++t) {
            double a = 0.0, b = 0.0;
            for (int i = 0; i < 128; ++i) {
                a += qh[i] * f64_from_canon(k_exact[t * 128 + i]);
                b += qh[i] * K[t * 128 + i];
            }
            se[t] = sigma * a;
            sq[t] = sigma * b;
            if (se[t] > Me) Me = se[t];
            if (sq[t] > Mq) Mq = sq[t];
        }
        /* log-normalizers of both distributions */
        double Le = 0.0, Lq = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            Le += exp(se[t] - Me);
            Lq += exp(sq[t] - Mq);
        }
        const double lse_e = Me + log(Le), lse_q = Mq + log(Lq);
        /* sum_t P_t (log P_t - log Q_t) */
        double acc = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            const double lp = se[t] - lse_e, lq = sq[t] - lse_q;
            acc += exp(lp) * (lp - lq);
        }
        kld[h] = acc;
    }
    free(K);
    free(se);
    free(sq);
    return 0;
}

/* ======================================================================== */
/* Chunked prefill attention (causal, over the mixed cache)                 */
/* ======================================================================== */

int kvo_prefill_attention(int64_t n, int64_t n_q, int64_t n_new, int fmt_k, int fmt_v,
                          const uint8_t* kq_codes, const uint16_t* kq_scales, const uint16_t* kq_cscale,
                          const uint8_t* vq_codes, const uint16_t* vq_scales, const uint16_t* vq_cscale,
                          const uint16_t* k_tail, const uint16_t* v_tail,
                          int g, const double* q, double sigma, double* out)
{
    int Nk, kk, cbk, sbk, pbk, Nv, kv, cbv, sbv, pbv;
    if (kvo_format_info(fmt_k, &Nk, &kk, &cbk, &sbk, &pbk) != 0) return -1;
    if (kvo_format_info(fmt_v, &Nv, &kv, &cbv, &sbv, &pbv) != 0) return -1;
    if (n_new == 0) return -4;
    if (n < 0 || n_q < 0 || n_q > n || n_new < 0 || n_new > n || g <= 0) return -1;
    /* every token of the sequence as the cache holds it */
    double* K = (double*)malloc(sizeof(double) * (size_t)n * 128);
    double* V = (double*)malloc(sizeof(double) * (size_t)n * 128);
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    if (!K || !V || !s) { free(K); free(V); free(s); return -1; }
    if (n_q > 0) {
        kvo_dequant_stream(fmt_k, n_q, kq_codes, kq_scales, kq_cscale, K);
        kvo_dequant_stream(fmt_v, n_q, vq_codes, vq_scales, vq_cscale, V);
    }
    for (int64_t t = n_q; t < n; ++t) {
        for (int i = 0; i < 128; ++i) {
            K[t * 128 + i] = f64_from_canon(k_tail[(t - n_q) * 128 + i]);
            V[t * 128 + i] = f64_from_canon(v_tail[(t - n_q) * 128 + i]);
        }
    }
    for (int64_t qi = 0; qi < n_new; ++qi) {
        const int64_t ctx = n - n_new + qi + 1;          /* tokens 0 .. p_i */
        for (int h = 0; h < g; ++h) {
            const double* qh = q + (qi * g + h) * 128;
            double M = -INFINITY;
            for (int64_t t = 0; t < ctx; ++t) {
                double acc = 0.0;
                for (int i = 0; i < 128; ++i) acc += qh[i] * K[t * 128 + i];
                s[t] = sigma * acc;
                if (s[t] > M) M = s[t];
            }
            double l = 0.0, o[128];
            for (int i = 0; i < 128; ++i) o[i] = 0.0;
            for (int64_t t = 0; t < ctx; ++t) {
                const double p = exp(s[t] - M);
                l += p;
                for (int i = 0; i < 128; ++i) o[i] += p * V[t * 128 + i];
            }
            for (int i = 0; i < 128; ++i) out[(qi * g + h) * 128 + i] = o[i] / l;
        }
    }
    free(K);
    free(V);
    free(s);
    return 0;
}
