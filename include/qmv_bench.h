/*
 * qmv_bench.h - measurement kernels shipped with libqmv (not part of the
 * QMV product API). They give the reference points the QMV kernels are
 * judged against on the same GPU:
 *
 *   qmv_bench_stream_read   reads `bytes` of device memory once with 16-byte
 *                           loads, `unroll` (1, 2, 4, 8 or 16) per lane, all
 *                           issued before any is used, and folds them into
 *                           one word per block: the measured ceiling of a
 *                           read-only stream of that size.
 *   qmv_bench_copy          copies `bytes` (a plain copy of known size, for
 *                           calibrating hardware byte counters).
 *
 * Pointers are device pointers; `bytes` must be a multiple of 16 and buffers
 * 16-byte aligned. `sink` must hold 65536 uint32 (a word is written only
 * in the practically impossible case that the fold equals a fixed pattern). Asynchronous on `stream`. Returns 0 or a hipError_t.
 */
#ifndef QMV_BENCH_H
#define QMV_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int qmv_bench_stream_read(void* stream, const void* buf, int64_t bytes, uint32_t* sink,
                          int unroll);
int qmv_bench_copy(void* stream, const void* src, void* dst, int64_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* QMV_BENCH_H */
