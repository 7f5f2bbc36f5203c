/*
 * attn_bench.h -- measurement helpers exported by libattn.so beside the attention
 * entry points of attn.h.  They compute nothing of the attention path; bench.py
 * uses them to measure the floor a split-KV decode call is compared against
 * (the decode is bound by reading the cached keys and values once: pofe.ai page
 * "FlashAttention for inference: tiled prefill and split-KV decoding", section
 * "Decode: a different bottleneck").
 */
#ifndef ATTN_BENCH_H_
#define ATTN_BENCH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attn_bench_stream_read -- one kernel that reads the device buffers a and b
 * (bytes_each bytes each, 16-byte aligned, bytes_each a multiple of 16) once,
 * with 16-byte loads, grid-stride, on `workgroups` workgroups of 256 threads;
 * each wave of workgroup w writes one uint32 (the XOR of what it read) to
 * sink[4 * w + wave], so sink must hold 4 * workgroups words (4-byte aligned).
 * Asynchronous on `stream`.  Returns 0, -1 (NULL pointer), -2 (bad size or
 * alignment) or -7 (launch failed).  bytes_each == 0 does nothing.
 */
int attn_bench_stream_read(const void *a, const void *b, size_t bytes_each, int workgroups, uint32_t *sink,
                           void *stream);

/*
 * attn_bench_empty -- an empty kernel (one workgroup of 64 threads) on `stream`:
 * the cost of one more dependent launch.  Returns 0 or -7 (launch failed).
 */
int attn_bench_empty(void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BENCH_H_ */
