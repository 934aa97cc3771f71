/*
 * kvq_debug.h -- diagnostic entry point of libkvq.so.
 *
 * The device-side scalar conversions and IEEE operations the encoders rely on, exposed so
 * they can be compared exhaustively with a CPU on the same inputs: round-to-nearest-even
 * bf16, round-to-nearest-even binary16 with saturation to +-65504 (zero stored as +0),
 * the correctly rounded reciprocal 1.0f/x and the correctly rounded sqrtf(x).
 * Also a timing hook that brackets the split-K decode kernel alone with caller events.
 */
#ifndef KVQ_DEBUG_H
#define KVQ_DEBUG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* in: n float32 device values.  Outputs (device, n elements each, any may be NULL):
 * bf16_out, fp16_out (bit patterns), recip_out = 1.0f/in, sqrt_out = sqrtf(in).
 * Enqueued on `stream`; returns 0 (KV_OK), KV_EINVAL for n < 0 or a null input,
 * KV_EDEVICE if the launch fails. */
int kv_debug_convert(const float* in, int64_t n, uint16_t* bf16_out, uint16_t* fp16_out,
                     float* recip_out, float* sqrt_out, void* stream);

/* Measurement hook.  While set, every decode call (kv_decode_attn, kv_decode_attn_noalloc)
 * records `before` on its stream immediately before the split-K decode kernel and `after`
 * immediately after it, before the merge kernel, so that the two events bracket that one
 * kernel.  The events are the caller's (hipEvent_t handles, created by the caller, kept
 * alive while set); passing two nulls clears the hook.  Process-wide and not synchronized
 * with concurrent decode calls: meant for a single measuring thread.  Returns 0 (KV_OK), or
 * KV_EINVAL when exactly one of the two is null.  A failed record makes the decode call
 * return KV_EDEVICE. */
int kv_debug_decode_events(void* before, void* after);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_DEBUG_H */
