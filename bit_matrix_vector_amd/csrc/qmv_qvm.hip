// qvm: the transposed quantized product y[b, k] = sum_n x[b, n] * W[n, k],
// W in the same packed [N, K] layout the QMV reads ("mlx 1.0.0 -
// quantized_nax.h", `qouter`: each row n adds x[n] times its dequantized row,
// scale * q + bias per element). Compiled once per dtype (QVM_DT).
//
// Work split: a lane owns 8 consecutive output columns (codes 8*SC .. 8*SC+7
// of one 32-code unit, all under one scale group: groups and blocks are at
// least 16 codes), so its accumulators are 8 per batch row (B <= 8). A block
// of 4 waves covers 512 columns over one split of the rows; its waves take
// interleaved rows (wave w: rows r0 + w, r0 + w + 4, ...), every wave reading
// x[b, n] at the same row, with the next row's words and scales in flight
// while the current one is accumulated. The waves' partial sums meet in LDS
// and the block writes them, fp32, to its row split's slice of the workspace;
// a second kernel adds the splits in order, so the result does not depend on
// timing. For affine codes the bias term sum_n x[n] * bias[n, g] is kept once
// per lane (its 8 columns share the group) and added to each column.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv_common.h"
#include "qmv_device.h"

#ifndef QVM_DT
#error "QVM_DT must be defined"
#endif

namespace qmv {
namespace {

constexpr int kQvThreads = 256;
constexpr int kQvCols = 8 * 64;   // output columns per block

// code words a lane loads per row: 1 for 2/4-bit codes and E2M1, 2 otherwise
template <int FMT, int BITS> constexpr int qvm_words() {
    return (FMT == FMT_MXFP4 || FMT == FMT_NVFP4 || (FMT == FMT_AFFINE && (BITS == 2 || BITS == 4)))
               ? 1
               : 2;
}

template <int DT, int FMT, int BITS>
struct QvRow {
    uint32_t d[qvm_words<FMT, BITS>()];
    uint32_t s;          // raw scale (bits of T for affine, a byte otherwise)
    uint32_t b;          // raw bias (affine)
    float x[8];          // x[b, n] for the batch rows
};

template <int DT, int FMT, int BITS, int NB>
__global__ __launch_bounds__(kQvThreads) void qvm_kernel(QvmParams q) {
    using S = typename Store<DT>::S;
    constexpr int kW = qvm_words<FMT, BITS>();
    extern __shared__ __align__(16) float part[];   // [4 waves][NB][512]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t K = q.K, N = q.N;
    const int64_t ncol8 = K >> 3;
    const int64_t col8 = (int64_t)blockIdx.x * 64 + lane;
    const int64_t c8 = col8 < ncol8 ? col8 : ncol8 - 1;   // past the end: re-read the last group
    const int64_t u = c8 >> 2;
    const int sc = (int)(c8 & 3);
    const int64_t r0 = (int64_t)blockIdx.y * q.rows_per_split;
    const int64_t r1 = r0 + q.rows_per_split < N ? r0 + q.rows_per_split : N;

    // where this lane's 8 codes sit in a row: a 4-byte aligned word and a bit
    // offset into it; the second word (if used) is clamped to the row
    int64_t word0;
    int off;
    if constexpr (FMT == FMT_AFFINE) {
        const int64_t byte0 = u * 4 * BITS + (int64_t)sc * BITS;
        word0 = byte0 >> 2;
        off = (int)(byte0 & 3) * 8;
    } else if constexpr (FMT == FMT_MXFP8) {
        word0 = u * 8 + 2 * sc;
        off = 0;
    } else {
        word0 = u * 4 + sc;
        off = 0;
    }
    const int64_t row_words = q.row_bytes >> 2;
    const int64_t word1 = word0 + 1 < row_words ? word0 + 1 : row_words - 1;
    int64_t sidx;   // scale element of the lane's columns
    if constexpr (FMT == FMT_AFFINE) sidx = (u * 32 + sc * 8) / q.group;
    else if constexpr (FMT == FMT_NVFP4) sidx = 2 * u + (sc >> 1);
    else sidx = u;

    const S* x = static_cast<const S*>(q.x);
    auto load_row = [&](QvRow<DT, FMT, BITS>& r, int64_t n) __attribute__((always_inline)) {
        const uint32_t* wr = reinterpret_cast<const uint32_t*>(q.w + n * q.row_bytes);
        r.d[0] = wr[word0];
        if constexpr (kW == 2) r.d[1] = wr[word1];
        if constexpr (FMT == FMT_AFFINE) {
            r.s = Store<DT>::load_bits(static_cast<const S*>(q.scales) + n * q.sc_per_row + sidx);
            r.b = Store<DT>::load_bits(static_cast<const S*>(q.biases) + n * q.sc_per_row + sidx);
        } else {
            r.s = static_cast<const uint8_t*>(q.scales)[n * q.sc_per_row + sidx];
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) r.x[b] = Store<DT>::load(x + b * N + n);
    };

    float acc[NB][8];
    float bsum[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        bsum[b] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[b][c] = 0.0f;
    }
    auto consume = [&](const QvRow<DT, FMT, BITS>& r) __attribute__((always_inline)) {
        float v[8];
        float s;
        if constexpr (FMT == FMT_AFFINE) {
            const uint64_t w64 = kW == 2 ? ((uint64_t)r.d[1] << 32) | r.d[0] : r.d[0];
            constexpr uint32_t mask = (1u << BITS) - 1u;
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (float)((uint32_t)(w64 >> (off + j * BITS)) & mask);
            s = Store<DT>::bits_to_f32(r.s);
        } else if constexpr (FMT == FMT_MXFP8) {
            const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.d[0], 1.0f, false);
            const f32x2 bb = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.d[0], 1.0f, true);
            const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.d[kW - 1], 1.0f, false);
            const f32x2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.d[kW - 1], 1.0f, true);
            v[0] = a.x; v[1] = a.y; v[2] = bb.x; v[3] = bb.y;
            v[4] = c.x; v[5] = c.y; v[6] = e.x; v[7] = e.y;
            s = e8m0_to_f32(r.s);
        } else {
            decode_e2m1_8(r.d[0], v);
            if constexpr (FMT == FMT_NVFP4) {
                const f32x2 t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.s, 1.0f, false);
                s = t.x;
            } else {
                s = e8m0_to_f32(r.s);
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float xs = r.x[b] * s;
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[b][c] = fmaf(xs, v[c], acc[b][c]);
            if constexpr (FMT == FMT_AFFINE)
                bsum[b] = fmaf(r.x[b], Store<DT>::bits_to_f32(r.b), bsum[b]);
        }
    };

    // rows r0 + wave, r0 + wave + 4, ...: two in flight
    int64_t n = r0 + wave;
    if (n < r1) {
        QvRow<DT, FMT, BITS> A, Bq;
        load_row(A, n);
        load_row(Bq, n + 4 < r1 ? n + 4 : n);
        for (; n + 8 < r1; n += 8) {
            consume(A);
            load_row(A, n + 8);
            consume(Bq);
            load_row(Bq, n + 12 < r1 ? n + 12 : n + 8);
        }
        consume(A);
        if (n + 4 < r1) consume(Bq);
    }

    // the 4 waves' partials meet in LDS; the block adds them in wave order
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int c = 0; c < 8; ++c)
            part[(wave * NB + b) * kQvCols + lane * 8 + c] = acc[b][c] + bsum[b];
    __syncthreads();
    float* ws = q.ws + (int64_t)blockIdx.y * q.B * K;
    for (int e = threadIdx.x; e < NB * kQvCols; e += kQvThreads) {
        const int b = e / kQvCols;
        const int col = e - b * kQvCols;
        const int64_t k = (int64_t)blockIdx.x * kQvCols + col;
        if (k < K) {
            float t = part[(0 * NB + b) * kQvCols + col];
            t += part[(1 * NB + b) * kQvCols + col];
            t += part[(2 * NB + b) * kQvCols + col];
            t += part[(3 * NB + b) * kQvCols + col];
            ws[b * K + k] = t;
        }
    }
}

template <int DT>
__global__ void qvm_reduce_kernel(QvmParams q, int splits) {
    using S = typename Store<DT>::S;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= q.B * q.K) return;
    float t = 0.0f;
    for (int s = 0; s < splits; ++s) t += q.ws[(int64_t)s * q.B * q.K + i];
    if (q.format == FMT_NVFP4 && q.gscale) t *= *q.gscale;
    static_cast<S*>(q.y)[i] = Store<DT>::from_f32(t);
}

template <int DT, int FMT, int BITS>
int launch_qvm_f(const QvmParams& q, hipStream_t st) {
    const dim3 grid((unsigned)((q.K + kQvCols - 1) / kQvCols), (unsigned)q.splits);
    const size_t lds = (size_t)4 * q.B * kQvCols * sizeof(float);
    switch (q.B) {
#define QV_CASE(nb)                                                                     \
    case nb:                                                                            \
        hipLaunchKernelGGL((qvm_kernel<DT, FMT, BITS, nb>), grid, dim3(kQvThreads), lds, st, q); \
        break;
        QV_CASE(1) QV_CASE(2) QV_CASE(3) QV_CASE(4) QV_CASE(5) QV_CASE(6) QV_CASE(7) QV_CASE(8)
#undef QV_CASE
        default: return (int)hipErrorInvalidValue;
    }
    const int64_t n = q.B * q.K;
    hipLaunchKernelGGL((qvm_reduce_kernel<DT>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       st, q, q.splits);
    return (int)hipGetLastError();
}

}  // namespace

#define QVM_CAT2(a, b) a##b
#define QVM_CAT(a, b) QVM_CAT2(a, b)

int QVM_CAT(launch_qvm_dt_, QVM_DT)(const QvmParams& q, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (q.format) {
        case FMT_AFFINE:
            switch (q.bits) {
                case 2: return launch_qvm_f<QVM_DT, FMT_AFFINE, 2>(q, st);
                case 3: return launch_qvm_f<QVM_DT, FMT_AFFINE, 3>(q, st);
                case 4: return launch_qvm_f<QVM_DT, FMT_AFFINE, 4>(q, st);
                case 5: return launch_qvm_f<QVM_DT, FMT_AFFINE, 5>(q, st);
                case 6: return launch_qvm_f<QVM_DT, FMT_AFFINE, 6>(q, st);
                case 8: return launch_qvm_f<QVM_DT, FMT_AFFINE, 8>(q, st);
            }
            return (int)hipErrorInvalidValue;
        case FMT_MXFP4: return launch_qvm_f<QVM_DT, FMT_MXFP4, 4>(q, st);
        case FMT_NVFP4: return launch_qvm_f<QVM_DT, FMT_NVFP4, 4>(q, st);
        case FMT_MXFP8: return launch_qvm_f<QVM_DT, FMT_MXFP8, 8>(q, st);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace qmv
