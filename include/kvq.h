/*
 * kvq.h -- C ABI of libkvq.so: a mixed-precision quantized KV cache for single-GPU
 * decoding on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources are web pages, cited by title and section):
 *  - The KV cache stores, per layer and KV head, the key and value vector of every
 *    token processed so far; each new token adds one pair, so the cache grows
 *    linearly with the context ["Beellama и Beellama-kvarn: как выборочное
 *    квантование KV-кэша влияет на качество кода", section "Что такое Beellama и
 *    выборочное квантование KV-кэша"].  -> kv_append
 *  - Generating the next token reads all of that accumulated state; at long context
 *    this read is memory bound ["Форк beellama и KV-кванты kvarn на длинном контексте:
 *    что известно об ускорении в 2026 году", section "Длинный контекст меняет профиль
 *    нагрузки с вычислений на работу с памятью"].  -> kv_decode_attn
 *  - Precision tail: the newest N tokens stay in BF16 while positions 0..n-N use the
 *    chosen low-bit type ["Экспериментальные методы квантизации KV-кэша в BeeLLama.cpp
 *    v0.4.0: KVarN и precision tail", section "Как это работает: гибридное хранение
 *    кэша"].  -> the tail_tokens setting and kv_spill_tail
 *  - Key and value cache types are chosen separately (same page, section
 *    "Конфигурация KV-кэша: примеры для типовых сценариев").  -> fmt_k, fmt_v
 *  - Formats q2_0 ... q6_1 and the KVarN types (same page, section "Расширенная
 *    палитра квантизации: от q2_0 до q6_1"; "BeeLLama.cpp v0.4.0: KVarN, KV 정밀도
 *    테일 (precision tail), q2_0-q3_1", KLD table); KVarN = Walsh-Hadamard rotation of
 *    each vector plus Sinkhorn balancing of per-dimension scales before quantization
 *    ["Практическое руководство: запуск Bonsai-Ternary-27B на 120k токенах с менее чем
 *    10 ГБ VRAM", section "Решение: KVarN - структурированная квантизация KV-кэша из
 *    исследований KIVI и QuIP#"], normalized once at write time and never recomputed
 *    on read ("Экспериментальные методы ...", section "Практический выигрыш: точность
 *    без потери скорости").
 *  The pages fix none of the bit layouts; the exact encodings this library implements
 *  are: block = 32 consecutive dims; qN_0 symmetric with an fp16 scale from the signed
 *  max-magnitude element; qN_1 affine (fp16 step and fp16 min); kvarnN = unnormalized
 *  Walsh-Hadamard rotation, 8 Sinkhorn iterations over a page of 128 tokens, fp16
 *  channel scales per page, then qN_0 on the normalized values; kvarnN_1 = the same
 *  page normalization with qN_1 on the normalized values (the var-norm switch over an
 *  affine base type: "Экспериментальные методы ...", section "Конфигурация KV-кэша:
 *  примеры для типовых сценариев"); codes packed as a little-endian N-bit stream per
 *  token.
 *
 * Conventions for every call:
 *  - Ownership: the library never allocates or frees device memory.  The cache buffer,
 *    inputs, outputs and the decode workspace are caller-owned device memory (the one
 *    exception, kv_decode_attn_noalloc, uses a fixed array of the library's code object).  Host
 *    arrays (seq_ids, n_new) are read during the call only.
 *  - Asynchrony: device work is enqueued on `stream` (a hipStream_t passed as void*;
 *    NULL = the default stream) and the call returns after enqueueing.  Host metadata
 *    (token counts) advances at call time, in stream order.  Inputs must stay valid
 *    until the stream has passed the call.
 *  - Errors: a negative kv_status is returned synchronously.  On any validation error
 *    nothing is enqueued and no metadata changes.  A failed launch returns KV_EDEVICE
 *    (the metadata has then advanced; the cache contents are undefined).  Faults during
 *    execution surface at the caller's next synchronization.  No C++ exception crosses
 *    the ABI.  One handle must not be used from two threads at once.
 *  - GQA: query head h reads KV head h / (n_q_heads / n_kv_heads).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KV_BF16 = 0,
    KV_Q2_0, KV_Q2_1, KV_Q3_0, KV_Q3_1, KV_Q4_0, KV_Q4_1, KV_Q5_0, KV_Q5_1,
    KV_Q6_0, KV_Q6_1, KV_Q8_0, KV_Q8_1,
    KV_KVARN2, KV_KVARN3, KV_KVARN4, KV_KVARN5, KV_KVARN6, KV_KVARN8,
    KV_KVARN2_1, KV_KVARN3_1, KV_KVARN4_1, KV_KVARN5_1, KV_KVARN6_1, KV_KVARN8_1,
    KV_NUM_FORMATS
} kv_format;

typedef enum {
    KV_OK = 0,
    KV_EINVAL = -1,        /* bad argument: null pointer, index out of range, bad size */
    KV_ENOSPC = -2,        /* an append would exceed max_tokens */
    KV_EUNSUPPORTED = -3,  /* valid but not implemented combination (e.g. head_dim != 128) */
    KV_EEMPTY = -4,        /* decode of a sequence with no tokens */
    KV_EDEVICE = -5,       /* HIP launch or device-query failure */
    KV_ESIZE = -6          /* buffer or workspace smaller than required */
} kv_status;

/* Input dtypes of kv_append and of the decode query. */
enum { KV_IN_BF16 = 0, KV_IN_F32 = 1 };

typedef struct {
    int32_t n_layers;      /* >= 1 */
    int32_t n_kv_heads;    /* >= 1 */
    int32_t n_q_heads;     /* n_q_heads / n_kv_heads must be 4 (the decode, prefill and KL
                            * kernels are built for GQA groups of 4; other groups return
                            * KV_EUNSUPPORTED) */
    int32_t head_dim;      /* must be 128 */
    int32_t fmt_k, fmt_v;  /* kv_format of the key and value caches (may differ) */
    int32_t tail_tokens;   /* T: newest tokens kept at 16 bits (0 = quantize everything) */
    int32_t n_seqs;        /* sequences (batch slots) held by the cache */
    int64_t max_tokens;    /* capacity per sequence, in tokens */
    int32_t tail_dtype;    /* KV_TAIL_BF16 (0, default) or KV_TAIL_F16: the 16-bit type of the
                            * tail ring, and the canonical value every quantized row is encoded
                            * from ("Экспериментальные методы квантизации KV-кэша в BeeLLama.cpp
                            * v0.4.0", section "KV Cache Precision Tail": BF16 or F16).  An F16
                            * value is the binary16 nearest the input (ties to even), saturated
                            * to +-65504, zero as +0.  KV_TAIL_F16 excludes the bf16 format. */
    int32_t reserved;      /* 0 */
} kv_config;

enum { KV_TAIL_BF16 = 0, KV_TAIL_F16 = 1 };

typedef struct kv_cache kv_cache;   /* opaque host handle */

/* Device bytes the caller must provide to kv_cache_init for this configuration, or a
 * negative kv_status for an invalid configuration.  Host only; no device work. */
int64_t kv_cache_bytes(const kv_config* cfg);

/* Create a handle over caller-owned device memory `dev_mem` of `bytes` bytes (256-byte
 * aligned).  All sequences start empty.  The buffer's contents need not be initialized.
 * Returns KV_OK and sets *out, or KV_EINVAL / KV_EUNSUPPORTED / KV_ESIZE. */
int kv_cache_init(const kv_config* cfg, void* dev_mem, int64_t bytes, kv_cache** out);

/* Free the host handle (not the device buffer).  NULL is accepted. */
int kv_cache_destroy(kv_cache* cache);

/* Append n_new[i] tokens to sequence seq_ids[i] (i < n_seqs, distinct ids).
 * layer >= 0: k and v are [sum(n_new)][n_kv_heads][128] for that layer;
 * layer == -1: k and v are [n_layers][sum(n_new)][n_kv_heads][128] (all layers).
 * Tokens of sequence seq_ids[i] occupy rows [sum_{j<i} n_new[j], ...) in call order.
 * in_dtype: KV_IN_BF16 or KV_IN_F32.  Every appended value is first made canonical: with a
 * BF16 tail, bf16 input is copied and fp32 input rounded to bf16 (nearest even); with an
 * F16 tail (tail_dtype), both are rounded to binary16 (nearest even, saturated to +-65504,
 * zero as +0).  Tokens that fall below the tail boundary
 * n_q = max(n_q, G*floor(max(0, n-T)/G)) are encoded with the stream's format (G = 128
 * when a format is KVarN: whole pages, else 1), newer ones are written to the 16-bit ring.
 * Values must be finite, and their canonical form too (an fp32 input beyond the largest
 * bf16 rounds to infinity): the encodings are defined for finite values only, and a block
 * holding a NaN or an infinity gets unspecified codes and scales.
 * Errors: KV_EINVAL (bad layer/seq/ids/pointers/dtype), KV_ENOSPC (capacity), and with
 * layer == -1, KV_EINVAL if the layers of a sequence disagree on their token counts;
 * KV_EDEVICE if a launch fails. */
int kv_append(kv_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
              const int32_t* n_new, const void* k, const void* v, int32_t in_dtype,
              void* stream);

/* Bytes of decode workspace needed by kv_decode_attn for up to n_seqs sequences at any
 * length up to max_tokens.  The workspace holds the per-workgroup partial results of one
 * call; it needs no initialization, and calls that share one workspace must be ordered on
 * one stream (or synchronized). */
int64_t kv_decode_workspace_bytes(const kv_cache* cache, int32_t n_seqs);

/* Single-token decode attention for `layer` over sequences seq_ids[0..n_seqs).
 * q: [n_seqs][n_q_heads][128] of q_dtype (KV_IN_BF16 or KV_IN_F32); out: float32
 * [n_seqs][n_q_heads][128].  For query head h of sequence s, with KV head h/g:
 *   s_t = softmax_scale * q_h . k_t,  out_h = sum_t exp(s_t - max) v_t / sum_t exp(s_t - max)
 * over every token t < n of the sequence: dequantized rows t < n_q, BF16 ring rows after.
 * No mask and no positional transform (keys arrive position-encoded).  Reads the cache
 * only.  Errors: KV_EINVAL, KV_EEMPTY (a sequence with n == 0), KV_ESIZE (workspace),
 * KV_EUNSUPPORTED (more than 32 sequences in one call, or a split plan above 8192
 * workgroups), KV_EDEVICE (a launch failed or the device could not be queried). */
int kv_decode_attn(kv_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                   const void* q, int32_t q_dtype, float softmax_scale, float* out,
                   void* workspace, int64_t ws_bytes, void* stream);

/* kv_decode_attn without a workspace and without allocating device memory, for callers
 * that cannot allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments (less the workspace) and results as kv_decode_attn,
 * with which it shares its kernels.  The split partials go to a fixed array inside the
 * library: 1024 partials, 4,259,840 bytes per device, held from the first call on that
 * device until the process ends; the split plan is capped at 1024 workgroups (the fast
 * kernel's plans use one per compute unit, up to four per compute unit when many
 * sequences and KV heads are decoded together).  Errors: as kv_decode_attn, plus KV_ESIZE
 * when even the smallest plan (2 workgroups per sequence and KV head) exceeds the array,
 * KV_EDEVICE if the array cannot be located.  Every call on one device uses that same
 * array: calls that overlap on one device (other streams, other threads) race and must be
 * ordered by the caller. */
int kv_decode_attn_noalloc(kv_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                           const void* q, int32_t q_dtype, float softmax_scale, float* out,
                           void* stream);

/* Bytes of workspace needed by kv_prefill_attn for a chunk of n_new tokens at any length
 * up to max_tokens (per-split partial results; no initialization needed; calls sharing it
 * must be stream-ordered). */
int64_t kv_prefill_workspace_bytes(const kv_cache* cache, int32_t n_new);

/* Chunked-prefill attention for `layer` of one sequence: the chunk is the sequence's last
 * n_new tokens, already appended (kv_append).  Query i of the chunk (q: [n_new][n_q_heads]
 * [128] of q_dtype) sits at position p = n - n_new + i and attends causally to the tokens
 * t <= p as the cache holds them (dequantized rows t < n_q, BF16 ring rows after):
 *   out[i][h] = sum_{t<=p} exp(s_t - max) v_t / sum_{t<=p} exp(s_t - max),
 *   s_t = softmax_scale * q_ih . k_t,  KV head h / g;
 * out: float32 [n_new][n_q_heads][128].  The step on the other side of append: prefill and
 * decode are measured separately ("Форк beellama и KV-кванты kvarn на длинном контексте",
 * the section on how to compare builds).  Reads the cache only.  Errors: KV_EINVAL
 * (n_new < 1 or n_new > n), KV_EEMPTY (n == 0), KV_ESIZE (workspace), KV_EUNSUPPORTED
 * (a ring of 8,388,608 slots or more: 2 GiB of 16-bit rows per stream). */
int kv_prefill_attn(kv_cache* cache, int32_t layer, int32_t seq_id, int32_t n_new, const void* q,
                    int32_t q_dtype, float softmax_scale, float* out, void* workspace,
                    int64_t ws_bytes, void* stream);

/* Bytes of workspace needed by kv_attn_kld at any length up to max_tokens (partial
 * results of one call; no initialization needed; calls sharing it must be stream-ordered). */
int64_t kv_attn_kld_workspace_bytes(const kv_cache* cache);

/* Attention fidelity of the cache for one (sequence, layer): for every query head h,
 *   kld[h] = KL(P || Q) = sum_t P_t log(P_t / Q_t),
 *   P_t = softmax_t(softmax_scale * q_h . k_ref_t),  Q_t = softmax_t(softmax_scale * q_h . k_t)
 * over t < n, where k_ref holds the exact keys of every token and k_t the keys the cache
 * holds (dequantized rows t < n_q, BF16 ring rows after).  A model-free analogue of the
 * pages' KL-divergence quality measure ("BeeLLama.cpp v0.4.0: KVarN, KV 정밀도 테일
 * (precision tail), q2_0-q3_1", KLD table), on attention weights rather than output tokens.
 * q: [n_q_heads][128] of q_dtype; k_ref: device [n][n_kv_heads][128] BF16 (the canonical
 * keys the cache was filled from, token-major); kld: device float32 [n_q_heads].  Reads
 * the cache only.  Errors: KV_EINVAL, KV_EEMPTY (n == 0), KV_ESIZE (workspace). */
int kv_attn_kld(kv_cache* cache, int32_t layer, int32_t seq_id, const void* q, int32_t q_dtype,
                float softmax_scale, const void* k_ref, float* kld, void* workspace,
                int64_t ws_bytes, void* stream);

/* Spill the tail of one sequence: n_q = max(n_q, G*floor(max(0, n - keep_tokens)/G)),
 * encoding the BF16 ring rows that cross the boundary.  layer == -1: all layers.
 * 0 <= keep_tokens <= tail_tokens.  Errors: KV_EINVAL. */
int kv_spill_tail(kv_cache* cache, int32_t layer, int32_t seq_id, int32_t keep_tokens,
                  void* stream);

/* Token count n and quantized boundary n_q of (seq, layer).  Host only. */
int kv_seq_get(const kv_cache* cache, int32_t seq, int32_t layer, int64_t* n, int64_t* n_q);

/* Set (n, n_q) of (seq, layer) (layer == -1: all layers), e.g. to reset a sequence to
 * (0, 0) or to restore a checkpointed buffer.  Requires 0 <= n_q <= n <= max_tokens,
 * n_q a multiple of G and n - n_q <= ring capacity.  Host only. */
int kv_seq_set(kv_cache* cache, int32_t seq, int32_t layer, int64_t n, int64_t n_q);

/* Byte offsets, inside the device buffer, of one stream's arrays (is_v = 0 keys,
 * 1 values): offsets[0] codes [max_tokens][code_bytes], offsets[1] block scales
 * [max_tokens][4] fp16 d (qN_1: [max_tokens][4][2] {d, m}), offsets[2] KVarN channel
 * scales [max_tokens/128][128] fp16 (-1 if none), offsets[3] BF16 ring [R][128];
 * *ring_slots = R.  Host only; used to inspect the cache. */
int kv_stream_layout(const kv_cache* cache, int32_t seq, int32_t layer, int32_t kv_head,
                     int32_t is_v, int64_t offsets[4], int64_t* ring_slots);

/* Format properties: bits N (16 for bf16), code bytes and scale bytes per token,
 * channel-scale bytes per 128-token page.  Host only. */
int kv_format_info(int32_t fmt, int32_t* bits, int32_t* code_bytes, int32_t* scale_bytes,
                   int32_t* page_bytes);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
