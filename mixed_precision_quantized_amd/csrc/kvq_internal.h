// kvq_internal.h -- layout of the cache buffer and the argument blocks passed from the
// host library to the HIP kernels.  Plain C++ (no HIP types): included by the host-only
// translation unit and by the kernel translation units.
#pragma once

#include <stdint.h>

namespace kvq {

constexpr int kD = 128;          // head_dim
constexpr int kBlock = 32;       // dims per block scale
constexpr int kPage = 128;       // tokens per KVarN page (channel-scale row)
constexpr int kTailUnit = 32;    // tokens of the BF16 ring per decode work unit
constexpr int kMaxSeqsPerLaunch = 32;
constexpr int kMaxGroup = 8;     // query heads per KV head
constexpr int kNumFormats = 25;  // format ids 0..24 (the C ABI's kv_format)

// KIND_KVARN: rotated, Sinkhorn-normalized pages over a symmetric block quantizer;
// KIND_KVARN1: the same over an affine (step and minimum) block quantizer.
enum Kind : int32_t { KIND_BF16 = 0, KIND_Q0 = 1, KIND_Q1 = 2, KIND_KVARN = 3, KIND_KVARN1 = 4 };

// Page formats: values stored rotated with a per-page channel-scale row.  (constexpr
// functions are callable from device code as well.)
constexpr bool kind_paged(int k) { return k == KIND_KVARN || k == KIND_KVARN1; }
// Formats whose blocks carry a step and a minimum (16 scale bytes per token).
constexpr bool kind_affine(int k) { return k == KIND_Q1 || k == KIND_KVARN1; }

struct FormatDesc {
    int32_t bits;         // N (16 for bf16)
    int32_t kind;         // Kind
    int32_t code_bytes;   // per token: 16N, or 256 for bf16
    int32_t scale_bytes;  // per token: 8 (qN_0, kvarnN), 16 (qN_1, kvarnN_1), 0 (bf16)
    int32_t page_bytes;   // per 128-token page: 256 (kvarnN, kvarnN_1), else 0
};

// Byte layout of one stream (the K or V history of one (seq, layer, kv_head)).
// All offsets are relative to the start of the stream and 256-byte aligned.
struct StreamLayout {
    int64_t codes;        // [max_tokens_pad][code_bytes]
    int64_t scales;       // [max_tokens_pad][scale_bytes]
    int64_t cscale;       // [max_tokens_pad/128][128] fp16, or -1
    int64_t ring;         // [ring_slots][128] bf16
    int64_t bytes;        // total bytes of the stream
};

// Everything a kernel needs to address a stream.
struct CacheGeom {
    char* base;           // device buffer
    int64_t unit_bytes;   // bytes of one (seq, layer, kv_head): K stream then V stream
    int64_t v_offset;     // offset of the V stream inside a unit (= K stream bytes)
    StreamLayout k, v;
    int32_t fmt_k, fmt_v;
    int32_t n_layers, n_kv_heads, n_q_heads, group;
    int32_t ring_slots;   // R
    int32_t tail_f16;     // 16-bit type of the ring and of canonical values: 0 bf16, 1 binary16
};

// Per-sequence entry of an append launch.
struct AppendSeq {
    int32_t seq;          // cache sequence slot
    int32_t in_row0;      // first input row of this sequence
    int64_t n_old;        // tokens before the call
    int64_t n_new;        // tokens after the call
    int64_t nq_old;       // quantized boundary before
    int64_t nq_new;       // quantized boundary after
};

struct AppendArgs {
    CacheGeom g;
    const void* k_in;     // [layers_in][rows][H][128]
    const void* v_in;
    int32_t in_dtype;     // 0 bf16, 1 fp32
    int32_t layer0;       // first cache layer addressed
    int32_t layers_in;    // layers present in the input (1 or n_layers)
    int32_t rows;         // sum of n_new over the call (input rows per layer)
    int32_t n_seqs;
    int32_t pad_;
    AppendSeq seqs[kMaxSeqsPerLaunch];
};

// Per-sequence entry of a decode launch.
struct DecodeSeq {
    int32_t seq;          // cache sequence slot
    int32_t in_idx;       // index into q / out
    int64_t n;
    int64_t n_q;
    int32_t units_q;      // quantized work units (128-token pages)
    int32_t units_t;      // tail work units (32 tokens)
    int32_t splits_q;     // workgroups per kv head over the quantized region
    int32_t splits_t;     // workgroups per kv head over the BF16 ring
    int32_t wg_base;      // first partial of this sequence ([head][split] order)
    int32_t q_base;       // quantized workgroups of the sequences before this one
    int32_t t_base;       // ring workgroups of the sequences before this one
    int32_t pad_;
};

struct DecodeArgs {
    CacheGeom g;
    int32_t layer;
    int32_t n_seqs;
    int32_t units_per_wg;   // quantized pages per workgroup
    int32_t q_dtype;      // 0 bf16, 1 fp32
    float scale_log2;     // softmax_scale * log2(e)
    int32_t units_per_wg_t; // ring units per workgroup
    int32_t q_wgs;        // quantized workgroups of the launch (they come first)
    int32_t pad_;
    const void* q;        // [n_seqs][n_q_heads][128]
    float* out;           // [n_seqs][n_q_heads][128]
    float* partials;      // [max_wgs][kPartialFloats]
    DecodeSeq seqs[kMaxSeqsPerLaunch];
};

// Attention fidelity of one (sequence, layer): per query head, the KL divergence of the
// attention distribution over the cache's keys from the one over exact BF16 keys.
constexpr int kKldTokens = 2048;   // tokens per split of the KL kernel
struct KldArgs {
    CacheGeom g;
    int32_t layer, seq;
    int64_t n, n_q;
    int32_t q_dtype;      // 0 bf16, 1 fp32
    float scale;          // softmax scale (natural-log domain)
    int32_t splits;       // ceil(n / kKldTokens)
    int32_t pass;         // 0: c = E_P[D] per head into cref; 1: KL into out
    const void* q;        // [n_q_heads][128]
    const uint16_t* k_ref;   // [n][n_kv_heads][128] bf16
    float* partials;      // [n_kv_heads][splits][kMaxGroup][4]: m, l, A, B
    float* cref;          // [n_q_heads]
    float* out;           // [n_q_heads]
};
int launch_kld(const KldArgs& a, void* stream);               // split kernel + merge (kvq_decode.hip)

// Causal attention of a sequence's last n_new tokens over the cache that holds them.
constexpr int kPfQ = 32;           // query positions per prefill workgroup
constexpr int kPfKB = 32;          // keys per prefill block
struct PrefillArgs {
    CacheGeom g;
    int32_t layer, seq;
    int64_t n, n_q;       // tokens of the sequence (the chunk is the last n_new), quantized boundary
    int32_t n_new, q_dtype;
    float scale_log2;     // softmax_scale * log2(e)
    int32_t tiles;        // ceil(n_new / kPfQ)
    int32_t splits_q, splits_t;   // key splits over the quantized blocks / the ring blocks
    int32_t bps;          // kPfKB-token blocks per split of the quantized region
    int32_t bps_t;        // the same for the ring region
    const void* q;        // [n_new][n_q_heads][128]
    float* out;           // [n_new][n_q_heads][128]
    float* partials;      // [n_kv_heads][tiles][splits][4][kPfQ][kD + 2]: m, l, acc
};
int launch_prefill(const PrefillArgs& a, void* stream);          // kvq_prefill.hip

constexpr int kPartialFloats = kMaxGroup * (kD + 2);   // m, l, acc[128] per query head
constexpr int kMaxDecodeWGs = 8192;
constexpr int kScratchWGs = 1024;   // decode partials in the library's own device array

// Kernel launchers (implemented in the .hip translation units).  Return 0 on a
// successful launch, or the HIP error code.
int launch_append_encode(const AppendArgs& a, void* stream);   // qN / bf16 streams
int launch_append_kvarn(const AppendArgs& a, void* stream);    // KVarN pages
int launch_append_ring(const AppendArgs& a, void* stream);     // BF16 ring writes
int launch_decode(const DecodeArgs& a, int n_wgs, void* stream);        // split kernel + merge
int launch_decode_split(const DecodeArgs& a, int n_wgs, void* stream);  // partials only
int launch_merge(const DecodeArgs& a, void* stream);                    // kvq_merge.hip
int set_decode_events(void* before, void* after);                         // timing hook of launch_decode
int decode_wgs_per_cu(int fmt_k, int fmt_v, int group);        // occupancy of the decode kernel
// 4-bit fast path (kvq_decode_ws.hip), used by launch_decode when it applies.
bool decode_fast_supported(int fmt_k, int fmt_v);
int launch_decode_fast(const DecodeArgs& a, int n_wgs, void* stream);
int decode_fast_wgs_per_cu(int fmt_k, int fmt_v);
int device_cu_count();
// The decode partials array of the current device for callers that cannot allocate
// (kvq_merge.hip); its size in *bytes; null if the device or the array cannot be located.
void* decode_scratch(int64_t* bytes);

}  // namespace kvq
