/* Drives the oracle's C code through the sanitizer build: every format's stream encoder
 * and dequantizer on exact-size heap buffers, the KVarN page encoders, the transform and
 * the balancing on their own, the ring image, decode, prefill and KL attention with and
 * without a tail, and the argument checks.  Prints "ok" and exits 0 when every call
 * returns what it should. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvq_oracle.h"

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "line %d: %s\n", __LINE__, #c); fails = 1; } } while (0)

static uint64_t st = 0x243F6A8885A308D3ull;
static double unif(void)
{
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return (double)(st >> 11) * (1.0 / 9007199254740992.0);
}
static uint16_t bf16(double x)
{
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int main(void)
{
    const int64_t n = 300, nk = 256;        /* kvarn: whole pages */
    uint16_t* x = malloc(sizeof(uint16_t) * n * 128);
    for (int64_t i = 0; i < n * 128; ++i) x[i] = bf16((unif() - 0.5) * 6.0 * (i % 37 == 0 ? 15.0 : 1.0));
    for (int f = 0; f < 25; ++f) {
        int N, kind, cb, sb, pb;
        EXPECT(kvo_format_info(f, &N, &kind, &cb, &sb, &pb) == 0);
        const int paged = pb > 0;
        const int64_t nq = paged ? nk : n;
        uint8_t* codes = malloc((size_t)(nq * cb));
        uint16_t* scales = sb ? malloc((size_t)(nq * sb)) : NULL;
        uint16_t* cs = paged ? malloc((size_t)(nq / 128 * 256)) : NULL;
        EXPECT(kvo_encode_stream(f, nq, x, codes, scales, cs) == 0);
        double* dq = malloc(sizeof(double) * nq * 128);
        EXPECT(kvo_dequant_stream(f, nq, codes, scales, cs, dq) == 0);
        for (int64_t i = 0; i < nq * 128; ++i) EXPECT(isfinite(dq[i]));
        /* attention: quantized rows then a bf16 tail of n - nq (or 44) tokens */
        const int64_t nn = nq + 44;
        uint16_t* tail = malloc(sizeof(uint16_t) * 44 * 128);
        memcpy(tail, x, sizeof(uint16_t) * 44 * 128);
        double q[4 * 128], out[4 * 128], kld[4];
        for (int i = 0; i < 4 * 128; ++i) q[i] = unif() - 0.5;
        EXPECT(kvo_attention(nn, nq, f, f, codes, scales, cs, codes, scales, cs, tail, tail, 4, q, 0.088, out) == 0);
        for (int i = 0; i < 4 * 128; ++i) EXPECT(isfinite(out[i]));
        if (nq >= 44) {
            double* qp = malloc(sizeof(double) * 44 * 4 * 128);
            double* op = malloc(sizeof(double) * 44 * 4 * 128);
            for (int i = 0; i < 44 * 4 * 128; ++i) qp[i] = unif() - 0.5;
            EXPECT(kvo_prefill_attention(nn, nq, 44, f, f, codes, scales, cs, codes, scales, cs, tail, tail, 4, qp,
                                         0.088, op) == 0);
            free(qp);
            free(op);
        }
        uint16_t* exact = malloc(sizeof(uint16_t) * nn * 128);
        memcpy(exact, x, sizeof(uint16_t) * nq * 128);
        memcpy(exact + nq * 128, tail, sizeof(uint16_t) * 44 * 128);
        EXPECT(kvo_attention_kld(nn, nq, f, codes, scales, cs, exact, 4, q, 0.088, kld) == 0);
        EXPECT(kvo_attention(0, 0, f, f, codes, scales, cs, codes, scales, cs, tail, tail, 4, q, 0.088, out) == -4);
        EXPECT(kvo_attention(nn, nn + 1, f, f, codes, scales, cs, codes, scales, cs, tail, tail, 4, q, 0.088, out) == -1);
        if (paged) EXPECT(kvo_encode_stream(f, 100, x, codes, scales, cs) == -1);
        free(exact);
        free(tail);
        free(dq);
        free(codes);
        free(scales);
        free(cs);
    }
    /* the pieces on their own */
    float y[128], A[128 * 128], r2[128], c2[128];
    for (int i = 0; i < 128; ++i) y[i] = (float)(unif() - 0.5);
    kvo_fwht128_f32(y);
    for (int i = 0; i < 128 * 128; ++i) A[i] = (float)(unif() * unif());
    kvo_sinkhorn128(A, 8, r2, c2);
    for (int i = 0; i < 128; ++i) EXPECT(r2[i] > 0.0f && c2[i] > 0.0f);
    for (int N = 2; N <= 8; ++N) {
        if (N == 7) continue;
        uint8_t* codes = malloc((size_t)(128 * 16 * N));
        uint16_t* sc = malloc(sizeof(uint16_t) * 128 * 8);
        uint16_t* cs = malloc(sizeof(uint16_t) * 128);
        kvo_encode_page_kvarn(N, x, codes, sc, cs);
        kvo_encode_page_kvarn_q1(N, x, codes, sc, cs);
        free(codes);
        free(sc);
        free(cs);
    }
    /* ring image and the state machine */
    const int64_t R = kvo_ring_capacity(100, 128);
    EXPECT(R == 128 * ((100 + 127 + 127) / 128) || R > 0);
    uint16_t* ring = calloc((size_t)R * 128, sizeof(uint16_t));
    EXPECT(kvo_ring_image(n, kvo_nq_after(0, n, 100, 128), R, x, ring) == 0);
    EXPECT(kvo_ring_image(n, 0, R, x, ring) != 0);
    EXPECT(kvo_nq_after(0, n, 100, 1) == n - 100);
    free(ring);
    free(x);
    if (fails) return 1;
    printf("ok\n");
    return 0;
}
