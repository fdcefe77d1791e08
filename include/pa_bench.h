/*
 * pa_bench.h -- measurement aids exported by libpa.so beside the calls of
 * pa.h.  They are not part of the method: they give the same-chip ceiling
 * that the decode kernels are measured against.  Both read every byte they
 * are given exactly once with the decode kernels' load form (16 bytes per
 * lane, nontemporal), fold it into an XOR so that no load can be dropped,
 * and write one 32-bit word per workgroup into `sink` (device memory).
 * Asynchronous on `stream`; argument errors return PA_ERR_INVALID (codes
 * of pa.h) before anything is enqueued.
 */
#ifndef PA_BENCH_H
#define PA_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Number of workgroups (and sink words) pa_bench_stream_read uses for a
 * buffer of `bytes`: one per MiB, rounded up. */
int64_t pa_bench_stream_read_groups(size_t bytes);

/* Plain streaming read of `bytes` (a multiple of 16) at `buf` (device,
 * 16-byte aligned), one consecutive MiB per workgroup.  `sink` receives
 * pa_bench_stream_read_groups(bytes) words. */
int pa_bench_stream_read(const void *buf, size_t bytes, uint32_t *sink,
                         void *stream);

/* The decode access pattern without its arithmetic: for every sequence s
 * and KV head h, the K and V slabs (block_size x head_dim fp16) of blocks
 * block_tables[s][0 .. ceil(context_lens[s] / block_size) - 1], whole
 * blocks, in table order, on the decode kernel's schedule (1 KiB wave
 * loads, 4 K + 4 V loads per wave step, two steps in flight).  Arguments as
 * for pa_decode; a slab (block_size * head_dim * 2 bytes) must be a power
 * of two of at least 1 KiB; an id outside
 * [0, num_blocks) reads block 0.  `sink` receives num_seqs * num_kv_heads
 * words. */
int pa_bench_block_read(const void *k_cache, const void *v_cache,
                        const int32_t *block_tables, int32_t max_blocks_per_seq,
                        const int32_t *context_lens, int32_t num_seqs,
                        int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t num_blocks, uint32_t *sink,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BENCH_H */
