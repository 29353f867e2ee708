/*
 * gqa_bench.h -- measurement helpers shipped with the decode library.
 *
 * Not part of the attention method. The bandwidth-wall section of the llms.blog
 * GQA/MQA page says decode is bound by reloading the KV cache from HBM each step, so
 * the decode kernel is measured against what plain streaming reads achieve on the same
 * device; this helper measures that ceiling.
 */
#ifndef GQA_BENCH_H
#define GQA_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* the library is built with hidden visibility; these are its exported symbols */
#pragma GCC visibility push(default)

/*
 * gqa_bench_read_stream -- read `bytes` bytes of device memory at `buf` (16-byte
 * aligned, bytes a multiple of 16) with coalesced 16-byte loads and write one
 * 32-bit checksum word per workgroup into `sink` (device, at least 4 * 8192 bytes)
 * so the reads cannot be elided. Asynchronous on `stream` (hipStream_t).
 * Returns a gqa_status (INVALID_ARGUMENT for NULL/misaligned pointers or sizes).
 */
int gqa_bench_read_stream(const void* buf, size_t bytes, void* sink, void* stream);

/*
 * gqa_bench_read_stream_lds -- read `bytes` bytes at `buf` (16-byte aligned, a
 * multiple of 16) the way the decode kernel streams its cache, minus the compute:
 * `workgroups` persistent workgroups (the decode kernel uses two per CU) each read one
 * contiguous share in steps of `step_bytes` (16384: a K + V tile of the 64/128-wide
 * kernels; 32768: a tile of the 512-wide latent) of direct-to-LDS loads, one step in
 * flight. Asynchronous on `stream`. Returns a gqa_status (INVALID_ARGUMENT for another
 * step size).
 */
int gqa_bench_read_stream_lds(const void* buf, size_t bytes, int workgroups, int step_bytes, void* stream);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif
#endif /* GQA_BENCH_H */
