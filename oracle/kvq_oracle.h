/*
 * kvq_oracle.h -- plain, slow, single-threaded CPU oracle for the mixed-precision
 * quantized KV cache (low-bit block formats, KVarN, BF16 precision tail) and for
 * single-token decode attention over it.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link, load or
 * call this code: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or constant generator with
 * the HIP library; the two are compared on the same seeded inputs.
 *
 * Sources (web pages; cited by title and section):
 *  [P1] "Beellama и Beellama-kvarn: как выборочное квантование KV-кэша влияет на
 *       качество кода" (ai-manual.ru).
 *  [P2] "Экспериментальные методы квантизации KV-кэша в BeeLLama.cpp v0.4.0: KVarN и
 *       precision tail" (ai-manual.ru).
 *  [P3] "Форк beellama и KV-кванты kvarn на длинном контексте: что известно об
 *       ускорении в 2026 году" (ai-manual.ru).
 *  [P4] "Практическое руководство: запуск Bonsai-Ternary-27B на 120k токенах с менее
 *       чем 10 ГБ VRAM" (ai-manual.ru).
 *  [P5] "BeeLLama.cpp v0.4.0: KVarN, KV 정밀도 테일 (precision tail), q2_0-q3_1"
 *       (molayo1419.me; translation of the fork author's release post).
 *
 * The pages give names, intent and memory arithmetic but no formulas, bit layouts,
 * rounding rules or Sinkhorn details.  Every place where this oracle fixes what the
 * pages leave open is marked READING and is listed in the design notes.
 *
 * Numeric ground rules (READING): every encode step is IEEE binary32 with each
 * operation rounded to nearest-even, no FMA contraction, subnormals honoured,
 * correctly rounded '/' and sqrtf.  Build flags: -std=c11 -O2 -ffp-contract=off
 * -fno-fast-math on x86-64 (SSE2 arithmetic, no x87 excess precision).  Decode-side
 * values (dequantized elements, attention) are exact reals evaluated in binary64.
 *
 * Function status: every function below is pinned by CPU tests against closed forms,
 * hand-checked worked examples, library routines or brute force, except where its
 * comment says "parity unpinned".
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache formats.  [P2 §"Расширенная палитра квантизации: от q2_0 до q6_1"] and
 * [P5 §"추가적인 표준 KV 캐시 유형"] name q2_0 ... q6_1 as new types next to the
 * upstream q4_0/q5_0/q5_1/q8_0; [P5, KLD table] names kvarn2 ... kvarn8.  The numbering
 * is an interface value shared with the library's public header (same integers). */
enum {
    KVO_BF16 = 0,
    KVO_Q2_0, KVO_Q2_1, KVO_Q3_0, KVO_Q3_1, KVO_Q4_0, KVO_Q4_1, KVO_Q5_0, KVO_Q5_1,
    KVO_Q6_0, KVO_Q6_1, KVO_Q8_0, KVO_Q8_1,
    KVO_KVARN2, KVO_KVARN3, KVO_KVARN4, KVO_KVARN5, KVO_KVARN6, KVO_KVARN8,
    /* var-norm over the affine bases: KVarN with qN_1 as the inner quantizer */
    KVO_KVARN2_1, KVO_KVARN3_1, KVO_KVARN4_1, KVO_KVARN5_1, KVO_KVARN6_1, KVO_KVARN8_1,
    KVO_NUM_FORMATS
};
enum { KVO_KIND_BF16 = 0, KVO_KIND_Q0 = 1, KVO_KIND_Q1 = 2, KVO_KIND_KVARN = 3, KVO_KIND_KVARN1 = 4 };

#define KVO_D 128        /* head_dim; the only supported value */
#define KVO_BLOCK 32     /* block of consecutive dims sharing one scale (READING) */
#define KVO_PAGE 128     /* KVarN page: tokens sharing one channel-scale row (READING) */

/* ---- scalar conversions ------------------------------------------------------ */
/* bf16(x): round-to-nearest-even to an 8-bit significand.  Precondition: x finite. */
uint16_t kvo_bf16_from_f32(float x);
float    kvo_f32_from_bf16(uint16_t b);

/* The canonical 16-bit type of values passed to the encoders, the ring image and the
 * attention references: bf16 (0, the default) or binary16 (1, an F16 tail).  Process-wide. */
void kvo_set_canonical_f16(int on);
int  kvo_canonical_f16(void);
/* fp16s(x): round-to-nearest-even to binary16, then +-inf -> +-65504 (saturate);
 * a zero result is always stored as +0 (0x0000).  Precondition: x finite. */
uint16_t kvo_fp16s_from_f32(float x);
double   kvo_f64_from_fp16(uint16_t h);

/* ---- format table -------------------------------------------------------------- */
/* Returns 0 and fills the outputs for a valid format, -1 otherwise.
 *  bits: N (16 for bf16); kind: KVO_KIND_*; code_bytes: bytes of one token's code row
 *  (16N, or 256 for bf16); scale_bytes: bytes of one token's block-scale row (8 for
 *  qN_0 and kvarnN: 4 fp16 d; 16 for qN_1: 4 x {fp16 d, fp16 m}; 0 for bf16);
 *  page_bytes: channel-scale bytes per 128-token page (256 for kvarn, else 0). */
int kvo_format_info(int fmt, int* bits, int* kind, int* code_bytes, int* scale_bytes,
                    int* page_bytes);

/* ---- block encoders (one block of 32 fp32 values) ------------------------------- */
/* E0, symmetric qN_0 (READING of "q4_0 ... fp16 scale, symmetric"): scale from the
 * signed max-magnitude element, all 2^N levels used, offset 2^(N-1). */
void kvo_encode_block_q0(int N, const float x[32], uint16_t* d16, uint8_t u[32]);
/* E1, affine qN_1 "with min": d = (max-min)/(2^N-1), m = min. */
void kvo_encode_block_q1(int N, const float x[32], uint16_t* d16, uint16_t* m16, uint8_t u[32]);

/* PK: a token's 128 N-bit codes as a little-endian bitstream of 16N bytes: bit k of
 * code j is stream bit j*N+k, stream bit s is bit s%8 of byte s/8. */
void kvo_pack_codes(int N, const uint8_t u[128], uint8_t* out);
void kvo_unpack_codes(int N, const uint8_t* in, uint8_t u[128]);

/* ---- KVarN pieces [P4 §"Решение: KVarN ..." and §"Как преобразование Уолша-Адамара
 *      и Sinkhorn спасают качество при 4-битном сжатии"] ------------------------------ */
/* Unnormalized Sylvester Walsh-Hadamard transform of 128 fp32 values, in place,
 * butterfly stages h = 1, 2, 4, ..., 64 (each butterfly one fp32 add and one sub). */
void kvo_fwht128_f32(float y[128]);
/* Sinkhorn balancing of a 128x128 matrix of squares A[t][j] (t = token, j = channel,
 * token-major).  iters iterations of (row step, column step) on squared scales;
 * c2 starts at 1.  Outputs the final r2[128] (tokens) and c2[128] (channels). */
void kvo_sinkhorn128(const float* A, int iters, float r2[128], float c2[128]);
/* Encode one 128-token page of one stream with kvarnN.  X: [128][128] bf16 bits,
 * token-major.  Outputs codes [128][16N], scales [128][4] fp16 d, cscale[128] fp16. */
/* The same page encoding with qN_1 (affine: fp16 step and minimum per block, scales
 * [128][4][2] {d, m}) as the inner quantizer: var-norm over an _1 base ("Экспериментальные
 * методы квантизации KV-кэша в BeeLLama.cpp v0.4.0": var-norm as a switch over a cache
 * type, e.g. q2_1 with --cache-var-norm). */
void kvo_encode_page_kvarn_q1(int N, const uint16_t* X, uint8_t* codes, uint16_t* scales,
                              uint16_t* cscale);
void kvo_encode_page_kvarn(int N, const uint16_t* X, uint8_t* codes, uint16_t* scales,
                           uint16_t* cscale);

/* ---- token / stream encoders ------------------------------------------------------ */
/* One token of a bf16 (identity), qN_0 or qN_1 stream.  x: 128 bf16 bits. */
int kvo_encode_token(int fmt, const uint16_t* x, uint8_t* codes, uint16_t* scales);
/* Encode rows [0, n_q) of one stream from its canonical bf16 rows x[n_q][128].
 * kvarn requires n_q % 128 == 0.  codes: [n_q][code_bytes]; scales: [n_q][scale_bytes/2]
 * fp16; cscale: [n_q/128][128] fp16 (kvarn only, may be NULL otherwise).
 * Returns 0, or -1 on a bad argument. */
int kvo_encode_stream(int fmt, int64_t n_q, const uint16_t* x, uint8_t* codes,
                      uint16_t* scales, uint16_t* cscale);

/* ---- decode side (binary64) ----------------------------------------------------- */
/* Dequantize one token: codes/scales of that token; cscale_row = the 128 fp16
 * channel scales of its page (kvarn only).  kvarn: Yhat[j] = c[j]*d[j/32]*(u-2^(N-1)),
 * x = (1/128) H Yhat with H[i][j] = (-1)^popcount(i&j) applied as an explicit matrix. */
int kvo_dequant_token(int fmt, const uint8_t* codes, const uint16_t* scales,
                      const uint16_t* cscale_row, double out[128]);

/* ---- precision tail state machine [P2 §"Как это работает: гибридное хранение кэша"] -- */
/* Granule G: 128 if either stream is kvarn, else 1 (READING: KVarN pages). */
int64_t kvo_granule(int fmt_k, int fmt_v);
/* Ring capacity R = G*ceil((T+G-1)/G) (0 when T = 0 and G = 1). */
int64_t kvo_ring_capacity(int64_t tail_tokens, int64_t granule);
/* n_q after an append (keep = T) or a spill (keep = keep_tokens):
 * max(n_q, G*floor(max(0, n-keep)/G)).  n is the token count after the call. */
int64_t kvo_nq_after(int64_t n_q, int64_t n, int64_t keep, int64_t granule);
/* Write the ring image of one stream: slot p % R holds the bf16 row of token p for
 * n_q <= p < n; other slots are left untouched.  x: canonical rows [n][128]. */
int kvo_ring_image(int64_t n, int64_t n_q, int64_t R, const uint16_t* x, uint16_t* ring);

/* ---- decode attention reference ---------------------------------------------------- */
/* One (sequence, layer, KV head) unit with g query heads sharing it (GQA).
 * Tokens t < n_q come from the quantized rows (kq_* / vq_*), tokens n_q <= t < n from
 * the bf16 rows k_tail/v_tail, given in token order ([n-n_q][128]).
 * s_t = sigma * sum_i q[h][i]*k_t[i]; o[h] = sum_t e^(s_t-M) v_t / sum_t e^(s_t-M),
 * all in binary64.  q: [g][128] values; out: [g][128].  Returns 0, -1 on bad
 * arguments, -4 when n == 0. */
int kvo_attention(int64_t n, int64_t n_q, int fmt_k, int fmt_v,
                  const uint8_t* kq_codes, const uint16_t* kq_scales, const uint16_t* kq_cscale,
                  const uint8_t* vq_codes, const uint16_t* vq_scales, const uint16_t* vq_cscale,
                  const uint16_t* k_tail, const uint16_t* v_tail,
                  int g, const double* q, double sigma, double* out);

/* ---- chunked prefill attention -------------------------------------------------------- */
/* Causal attention of the last n_new tokens of a sequence over the cache that holds them:
 * query i (0 <= i < n_new) sits at position p_i = n - n_new + i and attends to the tokens
 * t <= p_i, each as the cache holds it (dequantized rows t < n_q from the encoding of the
 * whole quantized region, bf16 rows k_tail/v_tail for n_q <= t < n, given in token order).
 * q: [n_new][g][128] values; out: [n_new][g][128]; binary64, same formula as
 * kvo_attention per query.  Returns 0, -1 on bad arguments, -4 when n_new == 0. */
int kvo_prefill_attention(int64_t n, int64_t n_q, int64_t n_new, int fmt_k, int fmt_v,
                          const uint8_t* kq_codes, const uint16_t* kq_scales, const uint16_t* kq_cscale,
                          const uint8_t* vq_codes, const uint16_t* vq_scales, const uint16_t* vq_cscale,
                          const uint16_t* k_tail, const uint16_t* v_tail,
                          int g, const double* q, double sigma, double* out);

/* ---- attention fidelity --------------------------------------------------------------- */
/* Kullback-Leibler divergence of the attention distribution over the cache's keys from the
 * one over the exact keys, per query head (a model-free analogue of the KLD quality
 * measure of "BeeLLama.cpp v0.4.0: KVarN, KV 정밀도 테일 (precision tail), q2_0-q3_1", KLD
 * table):  P_t = softmax_t(sigma q_h . x_t) over the exact bf16 keys x (k_exact, all n
 * tokens, [n][128]),  Q_t = softmax_t(sigma q_h . k_t) over the dequantized rows t < n_q
 * and the exact rows after (the bf16 tail),  kld[h] = sum_t P_t (log P_t - log Q_t), in
 * binary64.  Returns 0, -1 on bad arguments, -4 when n == 0. */
int kvo_attention_kld(int64_t n, int64_t n_q, int fmt_k, const uint8_t* kq_codes,
                      const uint16_t* kq_scales, const uint16_t* kq_cscale,
                      const uint16_t* k_exact, int g, const double* q, double sigma, double* kld);

/* Convenience for tests: dequantize rows [0, n_q) of one stream to binary64
 * (out: [n_q][128]). */
int kvo_dequant_stream(int fmt, int64_t n_q, const uint8_t* codes, const uint16_t* scales,
                       const uint16_t* cscale, double* out);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_ORACLE_H */
