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
 *   qmv_bench_read_design   reads `bytes` once with one of 20 read designs,
 *                           to find the fastest single launch for a size:
 *                           0-5 one-shot grids (threads x loads per lane:
 *                           256x2, 256x4, 256x8, 512x4, 1024x2, 64x8), 6 the
 *                           256x4 grid in XCD-contiguous block order, 7-8
 *                           32 / 64 contiguous bytes per lane, 9-14
 *                           persistent grid-stride (256 threads; 4 loads per
 *                           iteration on 256/512/1024/2048 blocks, 8 loads on
 *                           256/512), 15-16 [rows][2048] row patterns (eight
 *                           lanes per 128-byte line; the 16x16 MFMA operand
 *                           layout; bytes a multiple of 32 KB), 17 the
 *                           one-row QMV's loads over [rows][2048] weight
 *                           bytes then [rows][128] scale bytes (two rows per
 *                           wave, 64 lanes x 16 bytes per row and a scale
 *                           byte per lane; bytes a multiple of 8 x 2176),
 *                           18-19 design 17 followed by the write a QMV
 *                           makes (each wave folds its bytes and writes one
 *                           4-byte word per row pair to `sink`, 2 bytes per
 *                           row; at most 131072 rows), 19 in the one-row
 *                           QMV's XCD-chunked block order.
 *   qmv_bench_copy          copies `bytes` (a plain copy of known size, for
 *                           calibrating hardware byte counters).
 *
 * Pointers are device pointers; `bytes` must be a multiple of 16 and buffers
 * 16-byte aligned. `sink` must hold 65536 uint32 (designs 0-17 write a word
 * only in the practically impossible case that the fold equals a fixed
 * pattern; 18-19 write rows / 2 words). Asynchronous on `stream`. Returns 0
 * or a hipError_t.
 */
#ifndef QMV_BENCH_H
#define QMV_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int qmv_bench_stream_read(void* stream, const void* buf, int64_t bytes, uint32_t* sink,
                          int unroll);
int qmv_bench_read_design(void* stream, const void* buf, int64_t bytes, uint32_t* sink,
                          int design);
int qmv_bench_copy(void* stream, const void* src, void* dst, int64_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* QMV_BENCH_H */
