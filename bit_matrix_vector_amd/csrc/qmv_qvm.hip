// qvm: the transposed quantized product y[b, k] = sum_n x[b, n] * W[n, k],
// W in the same packed [N, K] layout the QMV reads ("mlx 1.0.0 -
// quantized_nax.h", `qouter`: each row n adds x[n] times its dequantized row,
// scale * q + bias per element). Compiled once per dtype (QVM_DT).
//
// Work split. A block covers a tile of output columns over one split of the
// rows, its waves each walking a contiguous run of the split's rows.
//   B <= 2: a lane owns a whole 32-code unit (one 16-byte load of 4-bit codes
//   per row, 32 accumulators per batch row); 8 waves per block, each loading
//   a batch of 8 rows (codes, scales and x) before using any of it.
//   B > 2: a lane owns 8 columns of a unit (8 accumulators per batch row;
//   groups and blocks are at least 16 codes, so the 8 share one scale); 4
//   waves per block, the split's x rows staged in LDS as fp32, the next chunk
//   of rows in flight while the current one is accumulated.
// The waves' partial sums meet in LDS, one batch row at a time, and the block
// writes them, fp32, to its row split's slice of the workspace; a second
// kernel adds the splits in a fixed order, so the result does not depend on
// timing. For affine codes the bias term sum_n x[n] * bias[n, g] is kept once
// per lane and added to each column.

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
constexpr int kQvChunk = 8;       // rows per chunk of a wave (two chunks in flight)

// code words a lane loads per row: 1 for 2/4-bit codes and E2M1, 2 otherwise
template <int FMT, int BITS> constexpr int qvm_words() {
    return (FMT == FMT_MXFP4 || FMT == FMT_NVFP4 || (FMT == FMT_AFFINE && (BITS == 2 || BITS == 4)))
               ? 1
               : 2;
}

template <int FMT, int BITS>
struct QvRow {
    uint32_t d[qvm_words<FMT, BITS>()];
    uint32_t s;          // raw scale (bits of T for affine, a byte otherwise)
    uint32_t b;          // raw bias (affine)
};

// x rows [r0, r0 + rows) of the batch as fp32 [rows][NB] in LDS
template <int DT, int NB>
__device__ inline void qvm_stage_x(const QvmParams& q, int64_t r0, int rows, float* xs) {
    using S = typename Store<DT>::S;
    const S* x = static_cast<const S*>(q.x);
    for (int e = threadIdx.x; e < rows * NB; e += kQvThreads) {
        const int b = e / rows;
        const int r = e - b * rows;
        xs[r * NB + b] = Store<DT>::load(x + b * q.N + r0 + r);
    }
}

// B <= 2: lane = one 32-code unit, tile = 64 units; 8 waves per block, each
// loading a batch of 8 rows (codes, raw scales, raw x) before using any, with
// wave-uniform row bases and 32-bit lane offsets
constexpr int kQvUnitWaves = 8;
constexpr int kQvBatch = 8;
template <int DT, int FMT, int BITS, int NB>
__global__ __launch_bounds__(64 * kQvUnitWaves) void qvm_unit_kernel(QvmParams q, int glog2) {
    using F = Fmt<FMT, BITS>;
    using S = typename Store<DT>::S;
    constexpr int W = F::kWords;
    constexpr int kUnitBytes = 4 * W;
    constexpr int kTile = 64 * 32;
    constexpr int kHalf = kQvUnitWaves / 2;
    constexpr int RB = kQvBatch;
    // LDS: partial sums of half the waves [kHalf][kTile]
    extern __shared__ __align__(16) float lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t K = q.K;
    const int64_t units = K >> 5;
    const int64_t ul = (int64_t)blockIdx.x * 64 + lane;
    const int64_t uc = ul < units ? ul : units - 1;   // past the end: re-read the last unit
    const int64_t r0 = (int64_t)blockIdx.y * q.rows_per_split;
    const int64_t r1 = r0 + q.rows_per_split < q.N ? r0 + q.rows_per_split : q.N;
    const int rows = (int)(r1 - r0);
    // this wave's rows: a run of whole batches (local indices a .. a + cnt)
    const int rpw = ((rows + kQvUnitWaves - 1) / kQvUnitWaves + RB - 1) / RB * RB;
    const int a = wave * rpw;
    const int cnt = (a + rpw < rows ? a + rpw : rows) - a;   // may be <= 0
    const uint32_t lane_w = (uint32_t)uc * kUnitBytes;
    const S* xg = static_cast<const S*>(q.x);

    struct Row {
        uint32_t d[W];
        typename F::Raw r;
        uint32_t x[NB];   // raw x[b, n]
    };
    auto load_batch = [&](Row* rr, int i0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const int i = i0 + j < cnt ? i0 + j : cnt - 1;   // past the run: re-read its last row
            const int64_t n = r0 + a + i;                      // wave-uniform
            load_words<W>(q.w + n * q.row_bytes + lane_w, rr[j].d);
            const uint32_t so = (uint32_t)(n * q.sc_per_row * F::template elem_bytes<DT>());
            rr[j].r = F::template global_raw<DT>(static_cast<const uint8_t*>(q.scales),
                                                 static_cast<const uint8_t*>(q.biases), so,
                                                 (int)uc, glog2);
#pragma unroll
            for (int b = 0; b < NB; ++b) rr[j].x[b] = Store<DT>::load_bits(xg + b * q.N + n);
        }
    };

    float acc[NB][32];
    float bsum[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        bsum[b] = 0.0f;
#pragma unroll
        for (int c = 0; c < 32; ++c) acc[b][c] = 0.0f;
    }
    auto consume = [&](const Row& r) __attribute__((always_inline)) {
        const auto sc = F::template decode<DT>(r.r);
        float v[4][8];
        static_for<0, 4>([&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            F::template decode8<k>(r.d, v[k]);
        });
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float xb = Store<DT>::bits_to_f32(r.x[b]);
            float xlo, xhi;
            if constexpr (FMT == FMT_NVFP4) {
                xlo = xb * sc.lo;
                xhi = xb * sc.hi;
            } else {
                xlo = xhi = xb * sc.s;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[b][8 * k + j] = fmaf(k < 2 ? xlo : xhi, v[k][j], acc[b][8 * k + j]);
            if constexpr (FMT == FMT_AFFINE) bsum[b] = fmaf(xb, sc.b, bsum[b]);
        }
    };

    // whole batches in the loop (no per-row branch, so the compiler keeps the
    // accumulators in place); the scheduling barrier keeps every load of a
    // batch ahead of its first use
    const int nfull = cnt > 0 ? cnt / RB : 0;
    for (int c = 0; c < nfull; ++c) {
        Row rr[RB];
        load_batch(rr, c * RB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < RB; ++j) consume(rr[j]);
    }
    if (cnt > 0 && nfull * RB < cnt) {
        Row rr[RB];
        load_batch(rr, nfull * RB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < RB; ++j)
            if (nfull * RB + j < cnt) consume(rr[j]);
    }

    // the waves' partials meet in LDS, one batch row at a time: waves
    // kHalf.. write, waves 0..kHalf-1 add theirs in place, then the block adds
    // the kHalf sums in order
    float* part = lds;
    float* ws = q.ws + (int64_t)blockIdx.y * q.B * K;
    const int64_t k0 = (int64_t)blockIdx.x * kTile;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if (wave >= kHalf) {
#pragma unroll
            for (int c = 0; c < 32; c += 4)
                *reinterpret_cast<float4*>(part + (wave - kHalf) * kTile + lane * 32 + c) =
                    make_float4(acc[b][c] + bsum[b], acc[b][c + 1] + bsum[b],
                                acc[b][c + 2] + bsum[b], acc[b][c + 3] + bsum[b]);
        }
        __syncthreads();
        if (wave < kHalf) {
#pragma unroll
            for (int c = 0; c < 32; c += 4) {
                float4* p = reinterpret_cast<float4*>(part + wave * kTile + lane * 32 + c);
                const float4 o = *p;
                *p = make_float4((acc[b][c] + bsum[b]) + o.x, (acc[b][c + 1] + bsum[b]) + o.y,
                                 (acc[b][c + 2] + bsum[b]) + o.z, (acc[b][c + 3] + bsum[b]) + o.w);
            }
        }
        __syncthreads();
        for (int col = threadIdx.x; col < kTile; col += 64 * kQvUnitWaves) {
            if (k0 + col < K) {
                float t = part[col];
#pragma unroll
                for (int w = 1; w < kHalf; ++w) t += part[w * kTile + col];
                ws[b * K + k0 + col] = t;
            }
        }
        __syncthreads();
    }
}

// B > 2: lane = 8 columns of a unit, tile = 512 columns
template <int DT, int FMT, int BITS, int NB>
__global__ __launch_bounds__(kQvThreads) void qvm_kernel(QvmParams q) {
    using S = typename Store<DT>::S;
    constexpr int kW = qvm_words<FMT, BITS>();
    // LDS: x rows of the split as fp32 [rows][NB], then 4 x 512 floats where
    // the waves' partial sums meet
    extern __shared__ __align__(16) float lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t K = q.K, N = q.N;
    const int64_t ncol8 = K >> 3;
    const int64_t col8 = (int64_t)blockIdx.x * 64 + lane;
    const int64_t c8 = col8 < ncol8 ? col8 : ncol8 - 1;   // past the end: re-read the last group
    const int64_t u = c8 >> 2;
    const int sc = (int)(c8 & 3);
    const int64_t r0 = (int64_t)blockIdx.y * q.rows_per_split;
    const int64_t r1 = r0 + q.rows_per_split < N ? r0 + q.rows_per_split : N;
    const int rows = (int)(r1 - r0);
    float* xs = lds;
    float* part = lds + (q.rows_per_split * NB + 3) / 4 * 4;

    qvm_stage_x<DT, NB>(q, r0, rows, xs);

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

    // this wave's rows: a run of whole chunks (local indices a .. e)
    const int rpw = ((rows + 3) / 4 + kQvChunk - 1) / kQvChunk * kQvChunk;
    const int a = wave * rpw;
    const int cnt = (a + rpw < rows ? a + rpw : rows) - a;   // may be <= 0

    auto load_chunk = [&](QvRow<FMT, BITS>* r, int i0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kQvChunk; ++j) {
            const int i = i0 + j < cnt ? i0 + j : cnt - 1;   // past the run: re-read its last row
            const int64_t n = r0 + a + i;
            const uint32_t* wr = reinterpret_cast<const uint32_t*>(q.w + n * q.row_bytes);
            r[j].d[0] = wr[word0];
            if constexpr (kW == 2) r[j].d[1] = wr[word1];
            if constexpr (FMT == FMT_AFFINE) {
                r[j].s = Store<DT>::load_bits(static_cast<const S*>(q.scales) + n * q.sc_per_row + sidx);
                r[j].b = Store<DT>::load_bits(static_cast<const S*>(q.biases) + n * q.sc_per_row + sidx);
            } else {
                r[j].s = static_cast<const uint8_t*>(q.scales)[n * q.sc_per_row + sidx];
            }
        }
    };

    float acc[NB][8];
    float bsum[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        bsum[b] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[b][c] = 0.0f;
    }
    auto consume = [&](const QvRow<FMT, BITS>& r, int i) __attribute__((always_inline)) {
        float v[8];
        float s;
        if constexpr (FMT == FMT_AFFINE) {
            const uint64_t w64 = kW == 2 ? ((uint64_t)r.d[1] << 32) | r.d[0] : r.d[0];
            constexpr uint32_t mask = (1u << BITS) - 1u;
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (float)((uint32_t)(w64 >> (off + j * BITS)) & mask);
            s = Store<DT>::bits_to_f32(r.s);
        } else if constexpr (FMT == FMT_MXFP8) {
            const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.d[0], 1.0f, false);
            const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.d[0], 1.0f, true);
            const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.d[kW - 1], 1.0f, false);
            const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.d[kW - 1], 1.0f, true);
            v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
            v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
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
        const float* xr = xs + (a + i) * NB;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float xb = xr[b];
            const float xsb = xb * s;
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[b][c] = fmaf(xsb, v[c], acc[b][c]);
            if constexpr (FMT == FMT_AFFINE) bsum[b] = fmaf(xb, Store<DT>::bits_to_f32(r.b), bsum[b]);
        }
    };
    auto consume_chunk = [&](const QvRow<FMT, BITS>* r, int i0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kQvChunk; ++j)
            if (i0 + j < cnt) consume(r[j], i0 + j);
    };

    __syncthreads();   // x rows staged
    if (cnt > 0) {
        QvRow<FMT, BITS> A[kQvChunk], Bc[kQvChunk];
        load_chunk(A, 0);
        if (kQvChunk < cnt) load_chunk(Bc, kQvChunk);
        for (int i0 = 0; i0 < cnt; i0 += 2 * kQvChunk) {
            consume_chunk(A, i0);
            if (i0 + 2 * kQvChunk < cnt) load_chunk(A, i0 + 2 * kQvChunk);
            if (i0 + kQvChunk < cnt) consume_chunk(Bc, i0 + kQvChunk);
            if (i0 + 3 * kQvChunk < cnt) load_chunk(Bc, i0 + 3 * kQvChunk);
        }
    }

    // the 4 waves' partials meet in LDS, one batch row at a time; the block
    // adds them in wave order
    float* ws = q.ws + (int64_t)blockIdx.y * q.B * K;
    const int64_t k0 = (int64_t)blockIdx.x * kQvCols;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int c = 0; c < 8; ++c) part[wave * kQvCols + lane * 8 + c] = acc[b][c] + bsum[b];
        __syncthreads();
        for (int col = threadIdx.x; col < kQvCols; col += kQvThreads) {
            if (k0 + col < K) {
                float t = part[col];
                t += part[kQvCols + col];
                t += part[2 * kQvCols + col];
                t += part[3 * kQvCols + col];
                ws[b * K + k0 + col] = t;
            }
        }
        __syncthreads();
    }
}

// y = sum of the splits' partials in a fixed order: wave w of a block adds
// splits w, w + 16, ... of 64 outputs, then the 16 sums are added in wave order
constexpr int kRedWaves = 16;
template <int DT>
__global__ __launch_bounds__(64 * kRedWaves) void qvm_reduce_kernel(QvmParams q, int splits) {
    using S = typename Store<DT>::S;
    __shared__ float red[kRedWaves][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t BK = q.B * q.K;
    const int64_t i = (int64_t)blockIdx.x * 64 + lane;
    float t = 0.0f;
    if (i < BK) {
        // 8 loads in flight per pass; past the last split, re-read it and add nothing
        const float* p = q.ws + i;
        for (int s0 = wave; s0 < splits; s0 += 8 * kRedWaves) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int s = s0 + j * kRedWaves;
                v[j] = p[(int64_t)(s < splits ? s : splits - 1) * BK];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) t = s0 + j * kRedWaves < splits ? t + v[j] : t;
        }
    }
    red[wave][lane] = t;
    __syncthreads();
    if (wave == 0 && i < BK) {
        t = red[0][lane];
#pragma unroll
        for (int w = 1; w < kRedWaves; ++w) t += red[w][lane];
        if (q.format == FMT_NVFP4 && q.gscale) t *= *q.gscale;
        static_cast<S*>(q.y)[i] = Store<DT>::from_f32(t);
    }
}

template <int DT, int FMT, int BITS>
int launch_qvm_f(const QvmParams& q, hipStream_t st) {
    const int64_t xs_floats = (q.rows_per_split * q.B + 3) / 4 * 4;
    if (q.B <= 2) {
        const size_t lds = (size_t)(kQvUnitWaves / 2) * 2048 * sizeof(float);
        const dim3 grid((unsigned)(((q.K >> 5) + 63) / 64), (unsigned)q.splits);
        const dim3 block(64 * kQvUnitWaves);
        int glog2 = 0;
        if (FMT == FMT_AFFINE) glog2 = q.group == 128 ? 2 : (q.group == 64 ? 1 : 0);
        if (q.B == 1)
            hipLaunchKernelGGL((qvm_unit_kernel<DT, FMT, BITS, 1>), grid, block, lds, st, q, glog2);
        else
            hipLaunchKernelGGL((qvm_unit_kernel<DT, FMT, BITS, 2>), grid, block, lds, st, q, glog2);
    } else {
        const dim3 grid((unsigned)((q.K + kQvCols - 1) / kQvCols), (unsigned)q.splits);
        const size_t lds = (size_t)(xs_floats + 4 * kQvCols) * sizeof(float);
        switch (q.B) {
#define QV_CASE(nb)                                                                         \
    case nb:                                                                                \
        hipLaunchKernelGGL((qvm_kernel<DT, FMT, BITS, nb>), grid, dim3(kQvThreads), lds, st, q); \
        break;
            QV_CASE(3) QV_CASE(4) QV_CASE(5) QV_CASE(6) QV_CASE(7) QV_CASE(8)
#undef QV_CASE
            default: return (int)hipErrorInvalidValue;
        }
    }
    const int64_t n = q.B * q.K;
    hipLaunchKernelGGL((qvm_reduce_kernel<DT>), dim3((unsigned)((n + 63) / 64)), dim3(64 * kRedWaves),
                       0, st, q, q.splits);
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
