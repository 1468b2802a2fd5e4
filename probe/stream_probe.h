/*
 * stream_probe.h -- C ABI of libnf4probe.so, a measurement aid beside the
 * benchmark (not part of libnf4): a plain streaming kernel that reads two
 * device byte ranges once and writes out_words 32-bit words, the bytes a
 * product launch over packed weights moves (Trapetum overview, "The bandwidth
 * law").  Its launch time is the floor a product launch of the same bytes is
 * compared with.
 *
 * nf4_probe_stream: a, b device pointers (16-byte aligned; a_bytes a multiple
 * of 16, b_bytes any), out device uint32 [out_words] (overwritten with
 * arbitrary values), variant in [0, nf4_probe_variants()), stream a hipStream_t
 * as void*.  Enqueues one kernel and returns 0; -1 bad argument, -2 misaligned,
 * -3 bad variant or size, -5 launch failure.  Nothing is enqueued on error
 * (except -5).
 */
#ifndef NF4_PROBE_H
#define NF4_PROBE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif
int nf4_probe_variants(void);
int nf4_probe_stream(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes,
                     uint32_t *out, int64_t out_words, int variant, void *stream);
#ifdef __cplusplus
}
#endif
#endif
