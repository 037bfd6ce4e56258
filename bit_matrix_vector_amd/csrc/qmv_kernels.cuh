// QMV kernels for gfx950 (MI355X / CDNA4).
//
// y[b, n] = sum_k x[b, k] * dequant(W)[n, k]  for B <= 8 activation rows.
//
// The product is bound by HBM bandwidth: every packed weight byte is read
// once and used B times. The kernel therefore
//   * streams each weight row with dword-aligned vector loads (16 bytes per
//     lane for 4-bit codes), consecutive lanes on consecutive bytes, and
//     issues the next unit's loads before it computes the current one;
//   * stages x once per block in LDS (in its stored type, in a layout where
//     the 64 lanes of a wave read consecutive 16-byte chunks), then keeps each
//     lane's x slice in registers while it is reused for R rows;
//   * decodes codes in registers (bit-field extracts for affine codes, the
//     gfx950 FP4/FP8 converters for E2M1/E4M3) and accumulates in fp32;
//   * folds each 32-code unit with its scale: for affine,
//     scale * sum(x*q) + bias * sum(x), sum(x) taken over fp32-widened x
//     ("mlx 1.0.0 - quantized_nax.h" `qdot`; "ml-explore/mlx pull request
//     4516"), for the block-scaled formats scale * sum(x*e);
//   * reduces across the lanes of a row with DPP lane moves, converts to the
//     output type with round-to-nearest-even and stores only rows < N; rows
//     past N re-read row N-1 so the loop has no row-dependent branch
//     ("ml-explore/mlx pull request 4516": the fast-rows tail).
//
// Work split: a row is covered by a lane group of LPR lanes (16, 32 or 64,
// chosen from K so that no lane idles), unit u of the row going to lane
// u mod LPR. A lane group owns R consecutive rows (2 or 4); a 256-thread
// block owns 4 * (64 / LPR) * R rows. The lane -> unit map and the order of every sum
// depend on K only, so a row's result is the same bits whatever N, B, the
// tile or the slab split is (tail rows equal a padded call bit for bit; the
// gathered product equals a one-row call bit for bit).

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "qmv_common.h"
#include "qmv_device.h"

namespace qmv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

struct Geom {
    int lpr;        // lanes per row group (16, 32, 64)
    int lpr_log2;
    int ks;         // x slab length in elements (multiple of 32*lpr, or K)
    int glog2;      // scale elements per unit (scale_glog2)
    int rows_per_block;
    int sc_lds_off;  // byte offset of the staged scales in LDS
    int sc_aligned4; // scale rows can be copied in 4-byte words
    int tiles_per_block;  // gather: consecutive row tiles one block runs
    int out_rows;         // gather: output rows per tile (rows_per_block, or half
                          // of it when each lane group computes a gate/up pair)
};

// x rows of a tile. Contiguous rows (qmv) or rows picked by an index list
// held in LDS (gather); `row(b)` is called with a run-time b.
// x row accessors of a tile: row(b) is batch row b; load(b, k) issues the
// global loads of the 16-byte chunk of that row starting at element k (and of
// whatever its staging needs) and returns them as a Chunk; stage(b, k, c) is
// that chunk as it goes into LDS (each element of the block's rows is staged
// exactly once, by one thread); finish() runs in every thread after the
// tile's sums and before its stores; out(b, v) is row b's fp32 result before
// the final rounding.
template <class S> struct XContig {
    using Chunk = v4u;
    const S* x;
    int64_t K;
    __device__ const S* row(int b) const { return x + (int64_t)b * K; }
    __device__ Chunk load(int b, int64_t k) const {
        return *reinterpret_cast<const v4u*>(row(b) + k);
    }
    __device__ v4u stage(int, int64_t, const Chunk& c) const { return c; }
    __device__ void finish() const {}
    __device__ float out(int, float v) const { return v; }
};
template <class S> struct XListed {
    using Chunk = v4u;
    const S* x;
    const int64_t* off;  // LDS: element offset of each staged row
    __device__ const S* row(int b) const { return x + off[b]; }
    __device__ Chunk load(int b, int64_t k) const {
        return *reinterpret_cast<const v4u*>(row(b) + k);
    }
    __device__ v4u stage(int, int64_t, const Chunk& c) const { return c; }
    __device__ void finish() const {}
    __device__ float out(int, float v) const { return v; }
};
// Fused RMSNorm. The row's normalization r[b] = 1 / sqrt(mean_k x^2 + eps) is
// one scalar, so it multiplies the fp32 dot products at the end; element k
// enters LDS as RN_T(x[b, k] * gamma[k]) — the product of two T values is
// exact in fp32, so that is one rounding of the exact product. The squares
// are summed as the elements are staged (fp32, each thread in its staging
// order), then over lanes and waves in a fixed order in finish(), so every
// block of a launch forms the same r.
template <int DT, int NB> struct XNorm {
    using S = typename Store<DT>::S;
    const S* x;
    int64_t K;
    const S* gamma;   // [K], 16-byte aligned
    float eps;
    float* red;       // LDS [NB][kWaves]
    mutable float ss[NB];
    mutable float r[NB];
    // gamma is loaded with x, so both are in flight before the weights
    struct Chunk {
        v4u x, g;
    };
    __device__ const S* row(int b) const { return x + (int64_t)b * K; }
    __device__ Chunk load(int b, int64_t k) const {
        return Chunk{*reinterpret_cast<const v4u*>(row(b) + k),
                     *reinterpret_cast<const v4u*>(gamma + k)};
    }
    __device__ v4u stage(int b, int64_t, const Chunk& c) const {
        const v4u v = c.x;
        const v4u gv = c.g;
        const uint32_t xi[4] = {v.x, v.y, v.z, v.w};
        const uint32_t gi[4] = {gv.x, gv.y, gv.z, gv.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (Store<DT>::kBytes == 4) {
                const float xv = __uint_as_float(xi[j]);
                ss[b] = fmaf(xv, xv, ss[b]);
                o[j] = __float_as_uint(xv * __uint_as_float(gi[j]));
            } else {
                const float x0 = Store<DT>::bits_to_f32(xi[j] & 0xFFFFu);
                const float x1 = Store<DT>::bits_to_f32(xi[j] >> 16);
                ss[b] = fmaf(x0, x0, ss[b]);
                ss[b] = fmaf(x1, x1, ss[b]);
                const f32x2 p = {x0 * Store<DT>::bits_to_f32(gi[j] & 0xFFFFu),
                                 x1 * Store<DT>::bits_to_f32(gi[j] >> 16)};
                // the pair converts (round to nearest even) in one instruction
                if constexpr (DT == DT_BF16)
                    o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2_t));
                else
                    o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, f16x2_t));
            }
        }
        return v4u{o[0], o[1], o[2], o[3]};
    }
    __device__ void finish() const {
        const int lane = threadIdx.x & 63;
        const int wave = threadIdx.x >> 6;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float t = ss[b];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
            if (lane == 0) red[b * kWaves + wave] = t;
        }
        __syncthreads();
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float t = red[b * kWaves];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) t += red[b * kWaves + w];
            r[b] = 1.0f / sqrtf(t / (float)K + eps);
        }
    }
    __device__ float out(int b, float v) const { return v * r[b]; }
};

// LDS layout of a staged x row: the 8-value sub-chunk sc of unit u sits at
// element (sc * us + u) * 8 (us = units in the slab), so the lanes of a wave,
// which walk consecutive units, read consecutive 16 bytes.
__device__ inline int x_lds_slot(int e0, int us) {
    const int u = e0 >> 5;
    const int sub = (e0 >> 3) & 3;
    return (sub * us + u) * 8 + (e0 & 7);
}

// 16 bytes of x (8 values of a 16-bit type) as stored in LDS: reordered to
// pairs (x[k], x[k+4]) where the packed affine path expects them.
template <int FMT, int BITS, int DT>
__device__ inline v4u stage_vec(v4u v) {
    if constexpr (Packed<FMT, BITS, DT>::kPerm) {
        v4u r;
        r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // x4 | x0
        r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // x5 | x1
        r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // x6 | x2
        r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // x7 | x3
        return r;
    } else {
        return v;
    }
}

// Raw weight loads of one unit (32 codes) for the R rows of a lane group.
template <int FMT, int BITS, int R> struct UnitRaw {
    uint32_t d[R][Fmt<FMT, BITS>::kWords];
};

// One unit (32 codes) of R rows against NB staged x rows, folded into the
// row totals with its scales: fp32 accumulation, then scale * acc (+ bias *
// sum(x) for affine). `ul` is the unit's index within the staged slab of `us`
// units and `ks` elements per x row. Shared by every tile loop, so a row's
// result does not depend on which loop computed it.
template <int DT, int FMT, int BITS, int NB, int R>
__device__ inline void unit_fma(const UnitRaw<FMT, BITS, R>& u_raw,
                                const typename Fmt<FMT, BITS>::Scale (&scl)[R],
                                const typename Store<DT>::S* lds, int ul, int ks, int us,
                                float (&total)[R][NB]) {
    using F = Fmt<FMT, BITS>;
    float acc[R][NB];
    float sx[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        sx[b] = 0.0f;
#pragma unroll
        for (int i = 0; i < R; ++i) acc[i][b] = 0.0f;
    }
    static_for<0, 4>([&](auto sc_c) {
        constexpr int SC = decltype(sc_c)::value;
        if constexpr (Packed<FMT, BITS, DT>::kOn) {
            // packed 16-bit path: weight pairs against x pairs, 2 MACs per op
            uint32_t xp[NB][4];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const v4u v = *reinterpret_cast<const v4u*>(lds + b * ks + (SC * us + ul) * 8);
                xp[b][0] = v.x; xp[b][1] = v.y; xp[b][2] = v.z; xp[b][3] = v.w;
                if constexpr (F::kNeedsSumX) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) sx[b] = dot2<DT>(xp[b][k], pair_ones<DT>(), sx[b]);
                }
            }
#pragma unroll
            for (int i = 0; i < R; ++i) {
                uint32_t wp[4];
                F::template pairs<SC, DT>(u_raw.d[i], wp);
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int k = 0; k < 4; ++k) acc[i][b] = dot2<DT>(wp[k], xp[b][k], acc[i][b]);
            }
        } else {
            float xv[NB][8];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                lds_load8<DT>(lds + b * ks + (SC * us + ul) * 8, xv[b]);
                if constexpr (F::kNeedsSumX) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) sx[b] += xv[b][j];
                }
            }
#pragma unroll
            for (int i = 0; i < R; ++i) {
                float q[8];
                F::template decode8<SC>(u_raw.d[i], q);
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[i][b] = fmaf(q[j], xv[b][j], acc[i][b]);
            }
        }
        if constexpr (F::kTwoScales) {
            if constexpr (SC == 1) {
                // first half (codes 0..15) done: fold it with its own scale
#pragma unroll
                for (int i = 0; i < R; ++i)
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        total[i][b] = fmaf(scl[i].lo, acc[i][b], total[i][b]);
                        acc[i][b] = 0.0f;
                    }
            }
        }
    });

#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if constexpr (FMT == FMT_AFFINE) {
                // scale * sum(x*q) + bias * sum(x); on the packed path the
                // codes entered as 1 + q/16, so sum(x*q) = 16 (acc - sum(x))
                if constexpr (Packed<FMT, BITS, DT>::kOn)
                    total[i][b] = fmaf(16.0f * scl[i].s, acc[i][b] - sx[b],
                                       fmaf(scl[i].b, sx[b], total[i][b]));
                else
                    total[i][b] = fmaf(scl[i].s, acc[i][b],
                                       fmaf(scl[i].b, sx[b], total[i][b]));
            } else if constexpr (F::kTwoScales) {
                total[i][b] = fmaf(scl[i].hi, acc[i][b], total[i][b]);
            } else {
                total[i][b] = fmaf(scl[i].s, acc[i][b], total[i][b]);
            }
        }
}

// One block's tile: rows [row_base, row_base + rows_per_block) of one weight
// matrix against NB activation rows.
//
// Per slab of K: each thread first issues global loads for its first few
// 16-byte chunks of x, then the lane's raw weight and scale loads for its
// first two units; only then does it write the x chunks to LDS, which waits
// for the x loads alone (vector-memory counters retire in order, and x went
// out first). Scale bytes stay undecoded until the unit is computed, and the
// next unit's loads are issued under uniform branches before the current unit
// is consumed, so two units per lane are in flight at every point.
//
// kStream: the weights and scales are read once (plain QMV), so their loads
// carry the nontemporal hint. kShort: the caller guarantees one slab (K fits
// the stage), 4-byte-aligned scale segments and at most two units per lane
// per row; the tile then has no slab loop, no steady-state refill loop and no
// byte-wise scale copy, which the register allocation would otherwise carry
// (62 instead of 78 VGPRs for the MXFP4 bf16 one-row tile: 8 waves per SIMD
// instead of 6). The arithmetic, and so every result, is the same either way.
template <int DT, int FMT, int BITS, int NB, int R, bool kStream = false, bool kShort = false,
          class XR>
__device__ inline void qmv_tile(const LaunchParams& p, const Geom& g, int64_t row_base,
                                const uint8_t* __restrict__ w, const void* sc, const void* bi,
                                const XR& xr, typename Store<DT>::S* const (&yrow)[NB],
                                float gmul, typename Store<DT>::S* lds) {
    using F = Fmt<FMT, BITS>;
    using S = typename Store<DT>::S;
    using U = UnitRaw<FMT, BITS, R>;
    constexpr int W = F::kWords;
    constexpr int kUnitBytes = 4 * W;
    constexpr int kPerVec = 16 / Store<DT>::kBytes;   // x values per 16-byte chunk
    // x chunks per row and thread issued ahead of the weights. The short
    // tile needs at most two (16-bit x) or four (f32) per row; f32 rows take
    // four while B <= 2 (with more rows the 16 extra VGPRs cost occupancy).
    // Longer rows take eight per row for B <= 2, four for B <= 4, two beyond
    // (measured at K=14336: B=1 9.1 -> 8.2 us, B=2 14.2 -> 13.1 us); indices
    // past the row clamp to its last chunk.
    constexpr int kXAhead = kShort ? ((DT == DT_F32 && NB <= 2) ? 4 : 2)
                                   : (NB <= 2 ? 8 : NB <= 4 ? 4 : 2);
    constexpr int kScAhead = 2;                       // scale words per thread issued first

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = lane >> g.lpr_log2;
    const int gl = lane & (g.lpr - 1);
    const int lpr = g.lpr;
    const int groups_per_wave = 64 >> g.lpr_log2;
    const int64_t N = p.N;
    const int64_t K = p.K;
    const int64_t row0 = row_base + (int64_t)(wave * groups_per_wave + grp) * R;

    // Weight addresses: the block's first row (uniform, in scalar registers)
    // plus a 32-bit per-lane offset; tail rows re-read the last valid row.
    const uint8_t* wblk = w + row_base * p.row_bytes;
    uint32_t wo[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t r = row0 + i;
        wo[i] = (uint32_t)(((r < N ? r : N - 1) - row_base) * p.row_bytes);
    }

    float total[R][NB];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) total[i][b] = 0.0f;

    auto load_unit = [&](U& u_raw, int64_t u) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < R; ++i)
            load_words<W, kStream>(wblk + (wo[i] + (uint32_t)(u * kUnitBytes)), u_raw.d[i]);
    };

    // Staged scales: per array, per block row, the scale elements of the
    // slab's units (`seg` bytes), rows clamped to N-1 like the weights.
    constexpr int kEB = F::template elem_bytes<DT>();
    const int RB = g.rows_per_block;
    const int rl0 = (wave * groups_per_wave + grp) * R;   // block-local row of i = 0
    uint8_t* lds_sc = reinterpret_cast<uint8_t*>(lds) + g.sc_lds_off;

    auto compute_unit = [&](const U& u_raw, int ul, int ks, int us, int seg)
                            __attribute__((always_inline)) {
        typename F::Scale scl[R];
#pragma unroll
        for (int i = 0; i < R; ++i)
            scl[i] = F::template decode<DT>(
                F::template lds_raw<DT>(lds_sc + (rl0 + i) * seg, RB * seg, ul, g.glog2));
        unit_fma<DT, FMT, BITS, NB, R>(u_raw, scl, lds, ul, ks, us, total);
    };

    for (int64_t slab = 0; slab < (kShort ? (int64_t)1 : K); slab += g.ks) {
        const int ks = (int)((K - slab) < g.ks ? (K - slab) : g.ks);
        const int us = ks >> 5;                          // units in this slab
        const int iters = (us + lpr - 1) >> g.lpr_log2;  // per lane, uniform
        const int64_t u0 = slab >> 5;
        const int vec_per_row = ks / kPerVec;

        // (1) the first x chunks of this thread (activation row 0). Every
        // load below is unconditional: an index past the end is clamped to
        // the last valid chunk or unit (all such lanes read one address, so
        // it costs one cache line), which keeps the number of loads in flight
        // the same on every path and lets each wait name exactly the loads it
        // needs.
        // The first chunks of every activation row go out here, ahead of the
        // weights: a chunk issued after them could only be staged once the
        // weights had arrived (the counters retire in order), which put an
        // HBM round trip in front of the x staging (B=4: 16.6 -> 12.9 us).
        typename XR::Chunk xs[NB][kXAhead];
        static_for<0, NB>([&](auto b_c) {
            constexpr int b = decltype(b_c)::value;
            static_for<0, kXAhead>([&](auto j_c) {
                constexpr int j = decltype(j_c)::value;
                const int v = min(tid + j * kThreads, vec_per_row - 1);
                xs[b][j] = xr.load(b, slab + (int64_t)v * kPerVec);
            });
        });

        // (1b) the first words of the tile's scale segment (when the scale
        // rows are not 4-byte aligned these loads read x instead and are
        // discarded; the bytes are copied after the barrier-free part below)
        const int seg = (int)F::elem_of_unit(us, g.glog2) * kEB;   // bytes per row per array
        const int64_t e0 = F::elem_of_unit(u0, g.glog2);
        const int wpr = seg >> 2;
        const int nw = (kShort || g.sc_aligned4) ? F::kArrays * RB * wpr : 0;
        auto sc_src = [&](int c) __attribute__((always_inline)) {   // byte c of the segment copy
            const int per_arr = RB * seg;
            const int a = c / per_arr;
            const int rem = c - a * per_arr;
            const int rl = rem / seg;
            const int k = rem - rl * seg;
            const int64_t row = min(row_base + rl, N - 1);
            const uint8_t* base = (F::kArrays == 2 && a == 1) ? static_cast<const uint8_t*>(bi)
                                                              : static_cast<const uint8_t*>(sc);
            return base + (row * p.sc_per_row + e0) * kEB + k;
        };
        // When the slab covers whole rows (one slab), each array's segment for
        // the block is one contiguous range and a word's source needs no
        // division; a word past the array end (rows >= N) is clamped to its
        // last word.
        const bool whole_rows = kShort || g.ks >= K;
        const int64_t row_stride = p.sc_per_row * kEB;
        auto sc_word = [&](int c) __attribute__((always_inline)) {
            const uint8_t* q;
            if (whole_rows) {
                const int per_arr = RB * seg;
                const bool second = F::kArrays == 2 && 4 * c >= per_arr;
                const uint8_t* base = second ? static_cast<const uint8_t*>(bi)
                                             : static_cast<const uint8_t*>(sc);
                const int64_t off = row_base * row_stride + (second ? 4 * c - per_arr : 4 * c);
                const int64_t last = N * row_stride - 4;
                q = base + (off < last ? off : last);
            } else {
                q = sc_src(4 * c);
            }
            if constexpr (kStream)
                return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(q));
            else
                return *reinterpret_cast<const uint32_t*>(q);
        };
        uint32_t sw[kScAhead];
        static_for<0, kScAhead>([&](auto j_c) {
            constexpr int j = decltype(j_c)::value;
            if (nw > 0) {
                sw[j] = sc_word(min(tid + j * kThreads, nw - 1));
            } else {
                sw[j] = *reinterpret_cast<const uint32_t*>(xr.row(0) + slab);
            }
        });

        // (2) raw loads of the lane's first two units (rows clamped to N-1)
        U A, Bq;
        load_unit(A, u0 + min(gl, us - 1));
        load_unit(Bq, u0 + min(gl + lpr, us - 1));

        // (3) x chunks to LDS; the rest of each row (slabs longer than
        // kXAhead chunks per thread) is loaded and stored here
        static_for<0, NB>([&](auto b_c) {
            constexpr int b = decltype(b_c)::value;
            static_for<0, kXAhead>([&](auto j_c) {
                constexpr int j = decltype(j_c)::value;
                const int v = tid + j * kThreads;
                if (v < vec_per_row)
                    *reinterpret_cast<v4u*>(lds + b * ks + x_lds_slot(v * kPerVec, us)) =
                        stage_vec<FMT, BITS, DT>(xr.stage(b, slab + v * kPerVec, xs[b][j]));
            });
            for (int v = tid + kXAhead * kThreads; v < vec_per_row; v += kThreads)
                *reinterpret_cast<v4u*>(lds + b * ks + x_lds_slot(v * kPerVec, us)) =
                    stage_vec<FMT, BITS, DT>(xr.stage(
                        b, slab + v * kPerVec, xr.load(b, slab + (int64_t)v * kPerVec)));
        });
        // (3b) scale segment to LDS
        if (nw > 0) {
            static_for<0, kScAhead>([&](auto j_c) {
                constexpr int j = decltype(j_c)::value;
                const int c = tid + j * kThreads;
                if (c < nw) reinterpret_cast<uint32_t*>(lds_sc)[c] = sw[j];
            });
            for (int c = tid + kScAhead * kThreads; c < nw; c += kThreads)
                reinterpret_cast<uint32_t*>(lds_sc)[c] = sc_word(c);
        } else if constexpr (!kShort) {
            const int nbytes = F::kArrays * RB * seg;
            for (int c = tid; c < nbytes; c += kThreads) lds_sc[c] = *sc_src(c);
        }
        __syncthreads();

        // (4) two units in flight: compute one, then refill its buffer with
        // the unit two steps ahead. The steady-state body runs while at least
        // one more unit follows the pair in hand (a refill past the end is
        // clamped); the last one or two units are consumed by a load-free
        // epilogue, so no wave ends waiting on loads it does not use.
        int it = 0;
        if constexpr (!kShort) {
            for (; it + 2 < iters; it += 2) {
                const int ua = gl + it * lpr;
                const int ub = ua + lpr;
                if (ua < us) compute_unit(A, ua, ks, us, seg);
                load_unit(A, u0 + min(ua + 2 * lpr, us - 1));
                if (ub < us) compute_unit(Bq, ub, ks, us, seg);
                load_unit(Bq, u0 + min(ub + 2 * lpr, us - 1));
            }
        }
        {
            const int ua = gl + it * lpr;
            const int ub = ua + lpr;
            if (ua < us) compute_unit(A, ua, ks, us, seg);
            if (it + 1 < iters && ub < us) compute_unit(Bq, ub, ks, us, seg);
        }
        __syncthreads();  // LDS is restaged for the next slab
    }

    // reduce over the LPR lanes of each row group (result in its last lane)
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            total[i][b] = group_sum(total[i][b], lpr);
        }

    xr.finish();
    if (gl == lpr - 1) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t r = row0 + i;
            if (r < N) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    float v = xr.out(b, total[i][b]);
                    if constexpr (FMT == FMT_NVFP4) v = v * gmul;
                    yrow[b][r] = Store<DT>::from_f32(v);
                }
            }
        }
    }
}

template <int DT, int FMT, int BITS, int NB, int R, bool SHORT>
__global__ __launch_bounds__(kThreads) void qmv_kernel(LaunchParams p, Geom g) {
    using S = typename Store<DT>::S;
    extern __shared__ __align__(16) unsigned char smem[];
    S* lds = reinterpret_cast<S*>(smem);
    S* yrow[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) yrow[b] = static_cast<S*>(p.y) + b * p.N;
    const XContig<S> xr{static_cast<const S*>(p.x), p.K};
    const float gmul = (FMT == FMT_NVFP4 && p.gscale) ? *p.gscale : 1.0f;
    qmv_tile<DT, FMT, BITS, NB, R, true, SHORT>(p, g, (int64_t)blockIdx.x * g.rows_per_block, p.w,
                                                p.scales, p.biases, xr, yrow, gmul, lds);
}

// Fused RMSNorm + QMV: y[b] = r[b] * (W . RN_T(x[b] * gamma)), the QMV tile
// with the XNorm accessor (x times gamma staged, the squares summed on the
// way, r applied to each row's result).
template <int DT, int FMT, int BITS, int NB, int R, bool SHORT>
__global__ __launch_bounds__(kThreads) void qmv_norm_kernel(LaunchParams p, Geom g, NormArgs na) {
    using S = typename Store<DT>::S;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float red[NB * kWaves];
    S* lds = reinterpret_cast<S*>(smem);
    XNorm<DT, NB> xr{static_cast<const S*>(p.x), p.K, static_cast<const S*>(na.gamma), na.eps,
                     red, {}, {}};
    S* yrow[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) yrow[b] = static_cast<S*>(p.y) + b * p.N;
    const float gmul = (FMT == FMT_NVFP4 && p.gscale) ? *p.gscale : 1.0f;
    qmv_tile<DT, FMT, BITS, NB, R, true, SHORT>(p, g, (int64_t)blockIdx.x * g.rows_per_block, p.w,
                                                p.scales, p.biases, xr, yrow, gmul, lds);
}

// ---------------------------------------------------------------------------
// Routed-expert gather. Grid (tile groups, n_experts + 1). Block (t, e) finds
// the slots routed to expert e (a ballot scan over rhs_indices, in slot
// order) and runs its group of consecutive row tiles on chunks of up to two of
// those slots. When K fits one slab, a chunk's x rows are staged in LDS once
// and serve every tile of the group, so the scan and the x staging are paid
// once per group rather than once per tile. Each expert's weights come from
// HBM once per call (further chunks of the same tiles re-read them from L2).
// The extra column e = n_experts writes the zero rows of slots whose expert or
// x row is out of range.
// ---------------------------------------------------------------------------
// Slots per chunk. A kernel carries the register budget of its largest
// instantiated tile, so chunks stay at two activation rows (the tile of a
// one- or two-row QMV); an expert with more slots runs several chunks over the
// same tiles, whose weights the repeat reads find in L2.
constexpr int kGatherChunkMax = 2;
__host__ __device__ constexpr int gather_chunk_for(int) { return kGatherChunkMax; }
constexpr int kGatherStageBytes = 32 * 1024;

// Units in flight per lane in the gather tile loop.
constexpr int kGatherDepth = 2;

// Gather tile loop for a one-slab geometry, with the chunk's NB x rows
// already staged in LDS for all of K. Each lane group walks its R-row set in
// tiles tile0 .. tile_end-1 and, within each tile, its units, as one sequence:
// the weight words and raw scales of the next units come straight from
// global memory and stay in flight across tile boundaries, and no barrier is
// taken, so each wave moves on at its own pace. A row's units, their order and
// the final reduction are those of qmv_tile, so results match it bit for bit.
// Gather modes: plain rows, or (MODE 1, R = 2) a lane group computing the
// gate row (from w) and the up row (from w2) of one output row, whose epilogue
// stores the activation swiglu(gate, up) instead of the two projections.
constexpr int kGatherPlain = 0;
constexpr int kGatherSwiglu = 1;

// silu(clamp(g)) * clamp(u): clamp g from above and u on both sides when the
// clamp is positive; silu(g) = g / (1 + exp(-g)) (exp overflowing to infinity
// for very negative g gives the limit 0).
__device__ inline float swiglu_act(float g, float u, float c) {
    if (c > 1.0e-6f) {
        g = fminf(g, c);
        u = fminf(fmaxf(u, -c), c);
    }
    return g / (1.0f + expf(-g)) * u;
}

template <int MODE>
using MoeArgsOf = typename std::conditional<MODE == kGatherSwiglu, MoeArgs, NoMoeArgs>::type;

template <int DT, int FMT, int BITS, int NB, int R, int MODE = kGatherPlain>
__device__ inline void gather_tiles(const LaunchParams& p, const MoeArgsOf<MODE>& m,
                                    const Geom& g, int64_t tile0,
                                    int64_t tile_end, const uint8_t* __restrict__ w,
                                    const void* sc, const void* bi,
                                    typename Store<DT>::S* const (&yrow)[NB], float gmul,
                                    const typename Store<DT>::S* lds) {
    using F = Fmt<FMT, BITS>;
    using U = UnitRaw<FMT, BITS, R>;
    constexpr int W = F::kWords;
    constexpr int kUnitBytes = 4 * W;
    struct Item {
        U u;
        typename F::Raw raw[R];
    };

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> g.lpr_log2;
    const int gl = lane & (g.lpr - 1);
    const int lpr = g.lpr;
    const int64_t N = p.N;
    const int ks = (int)p.K;
    const int us = ks >> 5;
    const int iters = (us + lpr - 1) >> g.lpr_log2;   // >= 1 (K > 0)
    static_assert(MODE == kGatherPlain || R == 2, "a gate/up pair takes two rows");
    constexpr bool kPair = MODE == kGatherSwiglu;
    const int64_t RB = g.out_rows;   // output rows per tile
    const int64_t rofs = (int64_t)(wave * (64 >> g.lpr_log2) + grp) * (kPair ? 1 : R);
    const int64_t n_items = (tile_end - tile0) * iters;

    // Load cursor. Addresses are a per-tile base (uniform) plus 32-bit
    // per-lane row offsets, refreshed when the cursor enters a tile; rows past
    // N re-read row N-1 and units past the row end re-read its last unit, like
    // qmv_tile. The cursor stops at the last item (later loads repeat it).
    const int64_t sc_row_bytes = p.sc_per_row * F::template elem_bytes<DT>();
    const uint8_t* const sc8 = static_cast<const uint8_t*>(sc);
    const uint8_t* const bi8 = static_cast<const uint8_t*>(bi);
    // pair mode: row i = 1 comes from the second matrix (same layout)
    const uint8_t* w_of[2] = {w, w};
    const uint8_t* sc_of[2] = {sc8, sc8};
    const uint8_t* bi_of[2] = {bi8, bi8};
    if constexpr (kPair) {
        w_of[1] = m.w2;
        sc_of[1] = static_cast<const uint8_t*>(m.scales2);
        bi_of[1] = static_cast<const uint8_t*>(m.biases2);
    }
    constexpr int kBases = kPair ? 2 : 1;
    int64_t lt = tile0;
    int lit = 0;
    const uint8_t* wt[kBases];   // weights of the cursor tile's first row
    const uint8_t* st[kBases];   // its scales (and, for affine, biases at bt)
    const uint8_t* bt[kBases];
    uint32_t wro[R];     // lane's row offsets from those, in weight bytes
    uint32_t sro[R];     // and in scale bytes
    auto enter_tile = [&](int64_t t) __attribute__((always_inline)) {
        const int64_t first = t * RB;
        const int64_t lim = N - 1 - first;   // last valid row, tile-relative
#pragma unroll
        for (int m = 0; m < kBases; ++m) {
            wt[m] = w_of[m] + first * p.row_bytes;
            st[m] = sc_of[m] + first * sc_row_bytes;
            bt[m] = FMT == FMT_AFFINE ? bi_of[m] + first * sc_row_bytes : st[m];
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t r = rofs + (kPair ? 0 : i);
            const uint32_t rr = (uint32_t)(r < lim ? r : lim);
            wro[i] = rr * (uint32_t)p.row_bytes;
            sro[i] = rr * (uint32_t)sc_row_bytes;
        }
    };
    enter_tile(lt);
    auto load_next = [&](Item& x) __attribute__((always_inline)) {
        const int u = min(gl + lit * lpr, us - 1);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int m = kPair ? i : 0;
            load_words<W>(wt[m] + (wro[i] + (uint32_t)u * kUnitBytes), x.u.d[i]);
            x.raw[i] = F::template global_raw<DT>(st[m], bt[m], sro[i], u, g.glog2);
        }
        if (++lit == iters) {
            if (lt + 1 < tile_end) {
                lit = 0;
                enter_tile(++lt);
            } else {
                lit = iters - 1;
            }
        }
    };

    float total[R][NB];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) total[i][b] = 0.0f;
    int64_t ct = tile0;
    int cit = 0;
    auto consume = [&](const Item& x) __attribute__((always_inline)) {
        const int u = gl + cit * lpr;
        if (u < us) {
            typename F::Scale scl[R];
#pragma unroll
            for (int i = 0; i < R; ++i) scl[i] = F::template decode<DT>(x.raw[i]);
            unit_fma<DT, FMT, BITS, NB, R>(x.u, scl, lds, u, ks, us, total);
        }
        if (++cit == iters) {
            // tile done: reduce over the row group, store, restart
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int b = 0; b < NB; ++b) total[i][b] = group_sum(total[i][b], lpr);
            if (gl == lpr - 1) {
                if constexpr (kPair) {
                    const int64_t r = ct * RB + rofs;
                    if (r < N) {
#pragma unroll
                        for (int b = 0; b < NB; ++b) {
                            float gv = total[0][b], uv = total[1][b];
                            if constexpr (FMT == FMT_NVFP4) {
                                gv = gv * gmul;
                                uv = uv * (m.gscale2 ? *m.gscale2 : 1.0f);
                            }
                            yrow[b][r] = Store<DT>::from_f32(swiglu_act(gv, uv, m.act_clamp));
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        const int64_t r = ct * RB + rofs + i;
                        if (r < N) {
#pragma unroll
                            for (int b = 0; b < NB; ++b) {
                                float v = total[i][b];
                                if constexpr (FMT == FMT_NVFP4) v = v * gmul;
                                yrow[b][r] = Store<DT>::from_f32(v);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int b = 0; b < NB; ++b) total[i][b] = 0.0f;
            cit = 0;
            ++ct;
        }
    };

    // a ring of kGatherDepth items in flight; the last few are consumed by a
    // load-free epilogue
    Item ring[kGatherDepth];
    static_for<0, kGatherDepth>([&](auto j_c) { load_next(ring[decltype(j_c)::value]); });
    int64_t k = 0;
    for (; k + kGatherDepth < n_items; k += kGatherDepth) {
        static_for<0, kGatherDepth>([&](auto j_c) {
            constexpr int j = decltype(j_c)::value;
            consume(ring[j]);
            load_next(ring[j]);
        });
    }
    static_for<0, kGatherDepth>([&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        if (k + j < n_items) consume(ring[j]);
    });
}

template <int DT, int FMT, int BITS, int R, bool kOneSlab, int MODE>
__device__ inline void gather_chunk(const LaunchParams& p, const MoeArgsOf<MODE>& m,
                                    const Geom& g, int64_t tile0,
                                    int64_t tile_end, const uint8_t* w, const void* sc,
                                    const void* bi, float gmul, const uint32_t* list,
                                    const int64_t* xoff, int cnt,
                                    typename Store<DT>::S* lds) {
    using S = typename Store<DT>::S;
    constexpr int kPerVec = 16 / Store<DT>::kBytes;
    const XListed<S> xr{static_cast<const S*>(p.x), xoff};
    const int64_t RB = g.out_rows;
    auto run = [&](auto nb_c) {
        constexpr int NB = decltype(nb_c)::value;
        S* yrow[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) yrow[b] = static_cast<S*>(p.y) + (int64_t)list[b] * p.N;
        if constexpr (kOneSlab) {
            // one slab: stage the chunk's x rows (whole K) once for the group
            const int K = (int)p.K;
            const int us = K >> 5;
            const int vec_per_row = K / kPerVec;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const v4u* src = reinterpret_cast<const v4u*>(xr.row(b));
                for (int v = threadIdx.x; v < vec_per_row; v += kThreads)
                    *reinterpret_cast<v4u*>(lds + b * K + x_lds_slot(v * kPerVec, us)) =
                        stage_vec<FMT, BITS, DT>(src[v]);
            }
            __syncthreads();
            gather_tiles<DT, FMT, BITS, NB, R, MODE>(p, m, g, tile0, tile_end, w, sc, bi, yrow,
                                                     gmul, lds);
        } else {
            static_assert(MODE == kGatherPlain, "the paired mode needs one slab");
            for (int64_t t = tile0; t < tile_end; ++t)
                qmv_tile<DT, FMT, BITS, NB, R>(p, g, t * RB, w, sc, bi, xr, yrow, gmul,
                                               lds);
        }
    };
    if (cnt == 1)
        run(std::integral_constant<int, 1>{});
    else
        run(std::integral_constant<int, 2>{});
}

// kOneSlab: K > 0 and the geometry holds all of K in one slab (the launcher
// checks), so the group runs gather_tiles; otherwise qmv_tile per tile.
// MODE kGatherSwiglu: the fused gate/up projection of the routed-MoE block
// (slot s reads x row s / top_k; w / w2 are the gate / up matrices; the output
// is the activation, one row per slot).
template <int DT, int FMT, int BITS, int R, bool kOneSlab, int MODE = kGatherPlain>
__global__ __launch_bounds__(kThreads) void gather_kernel(LaunchParams p, Geom g,
                                                          MoeArgsOf<MODE> m) {
    using S = typename Store<DT>::S;
    extern __shared__ __align__(16) unsigned char smem[];
    S* lds = reinterpret_cast<S*>(smem);
    constexpr int kChunk = gather_chunk_for(DT);
    __shared__ uint32_t list[kChunk + kThreads];   // matching slots, in slot order
    __shared__ uint32_t xrow[kChunk + kThreads];   // their x rows
    __shared__ int64_t xoff[kChunk];
    __shared__ int wave_cnt[kWaves];
    __shared__ int count;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t RB = g.out_rows;
    const int64_t n_tiles = (p.N + RB - 1) / RB;
    const int64_t tile0 = (int64_t)blockIdx.x * g.tiles_per_block;
    // x row of slot s
    auto x_row_of = [&](int64_t s) __attribute__((always_inline)) {
        if constexpr (MODE == kGatherSwiglu)
            return (uint32_t)(s / m.top_k);
        else
            return p.lhs[s];
    };
    const int64_t tile_end =
        tile0 + g.tiles_per_block < n_tiles ? tile0 + g.tiles_per_block : n_tiles;
    const int64_t e = blockIdx.y;

    if (e == p.n_experts) {
        // Zero rows for slots with an out-of-range expert or x row: one thread
        // per slot, all slots checked at once; such slots are rare, so the
        // owning thread writes the group's rows of that slot itself.
        const int64_t r0 = tile0 * RB;
        const int64_t r1 = tile_end * RB < p.N ? tile_end * RB : p.N;
        for (int64_t s = tid; s < p.n_slots; s += kThreads) {
            const uint32_t ex = p.rhs[s];
            const uint32_t xrw = x_row_of(s);
            if ((int64_t)ex < p.n_experts && (int64_t)xrw < p.n_x_rows) continue;
            S* yr = static_cast<S*>(p.y) + s * p.N;
            for (int64_t r = r0; r < r1; ++r) yr[r] = Store<DT>::from_f32(0.0f);
        }
        return;
    }

    const uint8_t* w = p.w + e * p.N * p.row_bytes;
    const void* sc;
    const void* bi = nullptr;
    if constexpr (FMT == FMT_AFFINE) {
        sc = static_cast<const S*>(p.scales) + e * p.N * p.sc_per_row;
        bi = static_cast<const S*>(p.biases) + e * p.N * p.sc_per_row;
    } else {
        sc = static_cast<const uint8_t*>(p.scales) + e * p.N * p.sc_per_row;
    }
    const float gmul = (FMT == FMT_NVFP4 && p.gscale) ? *p.gscale : 1.0f;
    if constexpr (MODE == kGatherSwiglu) {
        // the up matrix of expert e (the gate matrix is w above)
        m.w2 = m.w2 + e * p.N * p.row_bytes;
        if constexpr (FMT == FMT_AFFINE) {
            m.scales2 = static_cast<const S*>(m.scales2) + e * p.N * p.sc_per_row;
            m.biases2 = static_cast<const S*>(m.biases2) + e * p.N * p.sc_per_row;
        } else {
            m.scales2 = static_cast<const uint8_t*>(m.scales2) + e * p.N * p.sc_per_row;
        }
    }

    auto run_chunk = [&](int cnt) {
        if (tid < cnt) xoff[tid] = (int64_t)xrow[tid] * p.K;
        __syncthreads();
        gather_chunk<DT, FMT, BITS, R, kOneSlab, MODE>(p, m, g, tile0, tile_end, w, sc, bi,
                                                       gmul, list, xoff, cnt, lds);
        __syncthreads();
    };

    if (tid == 0) count = 0;
    __syncthreads();
    for (int64_t base = 0; base < p.n_slots; base += kThreads) {
        const int64_t s = base + tid;
        // both indices are read together (clamped), so one round trip serves
        const int64_t si = s < p.n_slots ? s : p.n_slots - 1;
        const uint32_t ex = p.rhs[si];
        const uint32_t xr = x_row_of(si);
        const bool match = s < p.n_slots && (int64_t)ex == e && (int64_t)xr < p.n_x_rows;
        const uint64_t m = __ballot(match);
        const int before = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) wave_cnt[wave] = __popcll(m);
        __syncthreads();
        // count is read only here, between the barriers that bracket its
        // update by thread 0 below
        const int prev = count;
        int off = prev;
        for (int i = 0; i < wave; ++i) off += wave_cnt[i];
        if (match) {
            list[off + before] = (uint32_t)s;
            xrow[off + before] = xr;
        }
        int added = 0;
        for (int i = 0; i < kWaves; ++i) added += wave_cnt[i];
        __syncthreads();
        int cnt = prev + added;
        while (cnt >= kChunk) {
            run_chunk(kChunk);
            // move the leftovers to the front
            const int rest = cnt - kChunk;
            uint32_t v = 0, vx = 0;
            if (tid < rest) {
                v = list[kChunk + tid];
                vx = xrow[kChunk + tid];
            }
            __syncthreads();
            if (tid < rest) {
                list[tid] = v;
                xrow[tid] = vx;
            }
            __syncthreads();
            cnt = rest;
        }
        if (tid == 0) count = cnt;
        __syncthreads();
    }
    const int cnt = count;
    if (cnt > 0) run_chunk(cnt);
}

// ---------------------------------------------------------------------------
// Down projection of the routed-MoE block, summed over each token's slots:
// y[t] = sum_j r[t, j] * (W[e[t, j]] . mid[t * top_k + j]). Grid (tile groups,
// tokens). A block compacts its token's slots with an in-range expert (in slot
// order), stages their mid rows in LDS (all of K), then each lane group walks
// (tile, slot, unit) as one pipelined sequence: at a slot's end its partial
// row sums are scaled by the slot's router weight and added to the row
// totals; at a tile's end the totals are reduced over the lane group and
// stored. Slots with an out-of-range expert add nothing.
// ---------------------------------------------------------------------------
constexpr int kMaxTopK = 16;

template <int DT, int FMT, int BITS, int R>
__global__ __launch_bounds__(kThreads) void moe_down_kernel(LaunchParams p, Geom g, MoeArgs m) {
    using S = typename Store<DT>::S;
    using F = Fmt<FMT, BITS>;
    using U = UnitRaw<FMT, BITS, R>;
    constexpr int W = F::kWords;
    constexpr int kUnitBytes = 4 * W;
    constexpr int kPerVec = 16 / Store<DT>::kBytes;
    struct Item {
        U u;
        typename F::Raw raw[R];
    };
    extern __shared__ __align__(16) unsigned char smem[];
    S* lds = reinterpret_cast<S*>(smem);
    __shared__ uint32_t slot_e[kMaxTopK];
    __shared__ float slot_r[kMaxTopK];
    __shared__ uint32_t slot_j[kMaxTopK];
    __shared__ int n_valid;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t t = blockIdx.y;
    const int64_t N = p.N;
    const int K = (int)p.K;
    const int us = K >> 5;
    const int64_t RB = g.out_rows;
    const int64_t n_tiles = (N + RB - 1) / RB;
    const int64_t tile0 = (int64_t)blockIdx.x * g.tiles_per_block;
    const int64_t tile_end =
        tile0 + g.tiles_per_block < n_tiles ? tile0 + g.tiles_per_block : n_tiles;

    // (1) the token's valid slots, in slot order (wave 0, one lane per slot)
    if (wave == 0) {
        const int j = lane < m.top_k ? lane : (int)m.top_k - 1;
        const uint32_t e = p.rhs[t * m.top_k + j];
        const float r = m.route_w[t * m.top_k + j];
        const bool ok = lane < m.top_k && (int64_t)e < p.n_experts;
        const uint64_t m = __ballot(ok);
        const int pos = __popcll(m & ((1ull << lane) - 1ull));
        if (ok) {
            slot_e[pos] = e;
            slot_r[pos] = r;
            slot_j[pos] = (uint32_t)j;
        }
        if (lane == 0) n_valid = __popcll(m);
    }
    __syncthreads();
    const int nv = n_valid;

    // (2) their mid rows into LDS, row v at v * K in the unit-interleaved layout
    const int vec_per_row = K / kPerVec;
    for (int v = 0; v < nv; ++v) {
        const v4u* src = reinterpret_cast<const v4u*>(static_cast<const S*>(p.x) +
                                                      (t * m.top_k + slot_j[v]) * (int64_t)K);
        for (int c = tid; c < vec_per_row; c += kThreads)
            *reinterpret_cast<v4u*>(lds + v * K + x_lds_slot(c * kPerVec, us)) =
                stage_vec<FMT, BITS, DT>(src[c]);
    }
    __syncthreads();

    const int grp = lane >> g.lpr_log2;
    const int gl = lane & (g.lpr - 1);
    const int lpr = g.lpr;
    const int iters = (us + lpr - 1) >> g.lpr_log2;
    const int64_t rofs = (int64_t)(wave * (64 >> g.lpr_log2) + grp) * R;
    S* yrow = static_cast<S*>(p.y) + t * N;
    const float gmul = (FMT == FMT_NVFP4 && p.gscale) ? *p.gscale : 1.0f;

    if (nv == 0) {
        // no routed expert: the token's rows are zero
        if (gl == lpr - 1) {
            for (int64_t tt = tile0; tt < tile_end; ++tt)
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const int64_t r = tt * RB + rofs + i;
                    if (r < N) yrow[r] = Store<DT>::from_f32(0.0f);
                }
        }
        return;
    }

    const int64_t sc_row_bytes = p.sc_per_row * F::template elem_bytes<DT>();
    const int64_t w_mat = N * p.row_bytes;           // bytes of one expert's matrix
    const int64_t s_mat = N * sc_row_bytes;
    const uint8_t* const sc8 = static_cast<const uint8_t*>(p.scales);
    const uint8_t* const bi8 = static_cast<const uint8_t*>(p.biases);
    const int64_t n_items = (tile_end - tile0) * nv * iters;

    // load cursor over (tile, slot, unit); stops at the last item
    int64_t lt = tile0;
    int lv = 0, lit = 0;
    const uint8_t* wt;
    const uint8_t* st;
    const uint8_t* bt;
    uint32_t wro[R], sro[R];
    auto enter = [&]() __attribute__((always_inline)) {
        const int64_t first = lt * RB;
        const int64_t e = slot_e[lv];
        wt = p.w + e * w_mat + first * p.row_bytes;
        st = sc8 + e * s_mat + first * sc_row_bytes;
        bt = FMT == FMT_AFFINE ? bi8 + e * s_mat + first * sc_row_bytes : st;
        const int64_t lim = N - 1 - first;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t r = rofs + i;
            const uint32_t rr = (uint32_t)(r < lim ? r : lim);
            wro[i] = rr * (uint32_t)p.row_bytes;
            sro[i] = rr * (uint32_t)sc_row_bytes;
        }
    };
    enter();
    auto load_next = [&](Item& x) __attribute__((always_inline)) {
        const int u = min(gl + lit * lpr, us - 1);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            load_words<W>(wt + (wro[i] + (uint32_t)u * kUnitBytes), x.u.d[i]);
            x.raw[i] = F::template global_raw<DT>(st, bt, sro[i], u, g.glog2);
        }
        if (++lit == iters) {
            if (lv + 1 < nv) {
                lit = 0;
                ++lv;
                enter();
            } else if (lt + 1 < tile_end) {
                lit = 0;
                lv = 0;
                ++lt;
                enter();
            } else {
                lit = iters - 1;
            }
        }
    };

    float part[R][1], total[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        part[i][0] = 0.0f;
        total[i] = 0.0f;
    }
    int64_t ct = tile0;
    int cv = 0, cit = 0;
    auto consume = [&](const Item& x) __attribute__((always_inline)) {
        const int u = gl + cit * lpr;
        if (u < us) {
            typename F::Scale scl[R];
#pragma unroll
            for (int i = 0; i < R; ++i) scl[i] = F::template decode<DT>(x.raw[i]);
            unit_fma<DT, FMT, BITS, 1, R>(x.u, scl, lds + cv * K, u, K, us, part);
        }
        if (++cit == iters) {
            const float r = slot_r[cv];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                total[i] = fmaf(r, part[i][0], total[i]);
                part[i][0] = 0.0f;
            }
            cit = 0;
            if (++cv == nv) {
#pragma unroll
                for (int i = 0; i < R; ++i) total[i] = group_sum(total[i], lpr);
                if (gl == lpr - 1) {
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        const int64_t row = ct * RB + rofs + i;
                        if (row < N) yrow[row] = Store<DT>::from_f32(total[i] * gmul);
                    }
                }
#pragma unroll
                for (int i = 0; i < R; ++i) total[i] = 0.0f;
                cv = 0;
                ++ct;
            }
        }
    };

    Item ring[kGatherDepth];
    static_for<0, kGatherDepth>([&](auto j_c) { load_next(ring[decltype(j_c)::value]); });
    int64_t k = 0;
    for (; k + kGatherDepth < n_items; k += kGatherDepth) {
        static_for<0, kGatherDepth>([&](auto j_c) {
            constexpr int j = decltype(j_c)::value;
            consume(ring[j]);
            load_next(ring[j]);
        });
    }
    static_for<0, kGatherDepth>([&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        if (k + j < n_items) consume(ring[j]);
    });
}

// ---------------------------------------------------------------------------
// Device codecs: the same extraction and decoders as the kernels above.
// One thread per (row, unit of 32 codes).
// ---------------------------------------------------------------------------
template <int BITS>
__global__ void unpack_kernel(const uint8_t* __restrict__ packed, int64_t rows, int64_t K,
                              uint8_t* __restrict__ codes) {
    const int64_t units = K >> 5;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= rows * units) return;
    const int64_t r = t / units, u = t % units;
    uint32_t d[BITS];
    load_words<BITS>(packed + r * (K * BITS / 8) + u * 4 * BITS, d);
    uint8_t* out = codes + r * K + u * 32;
#pragma unroll
    for (int j = 0; j < 32; ++j) out[j] = (uint8_t)affine_code<BITS>(d, j);
}

template <int FMT, int BITS, int SC, class Sc>
__device__ inline float dequant_value(const Sc& s, float q, float gmul) {
    if constexpr (FMT == FMT_AFFINE) return fmaf(s.s, q, s.b);
    else if constexpr (Fmt<FMT, BITS>::kTwoScales) return (q * (SC < 2 ? s.lo : s.hi)) * gmul;
    else return q * s.s;
}

template <int DT, int FMT, int BITS>
__global__ void dequant_kernel(LaunchParams p, int glog2, float* __restrict__ out) {
    using F = Fmt<FMT, BITS>;
    constexpr int W = F::kWords;
    const int64_t units = p.K >> 5;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= p.N * units) return;
    const int64_t r = t / units, u = t % units;
    uint32_t d[W];
    load_words<W>(p.w + r * p.row_bytes + u * 4 * W, d);
    const typename F::Scale s =
        F::template decode<DT>(
            F::template load_raw<DT>(p.scales, p.biases, r, p.sc_per_row, u, glog2));
    const float gmul = (FMT == FMT_NVFP4 && p.gscale) ? *p.gscale : 1.0f;
    float* o = out + r * p.K + u * 32;
    static_for<0, 4>([&](auto sc_c) {
        constexpr int SC = decltype(sc_c)::value;
        float q[8];
        if constexpr (Packed<FMT, BITS, DT>::kOn) {
            // decode through the packed pairs the QMV kernel uses for this dtype
            uint32_t wp[4];
            F::template pairs<SC, DT>(d, wp);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float lo = F::pair_code(pair_lo<DT>(wp[k]));
                const float hi = F::pair_code(pair_hi<DT>(wp[k]));
                if constexpr (Packed<FMT, BITS, DT>::kPerm) {
                    q[k] = lo;
                    q[k + 4] = hi;
                } else {
                    q[2 * k] = lo;
                    q[2 * k + 1] = hi;
                }
            }
        } else {
            F::template decode8<SC>(d, q);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            o[SC * 8 + j] = dequant_value<FMT, BITS, SC>(s, q[j], gmul);
        }
    });
}

// ---------------------------------------------------------------------------
// Host-side launch helpers.
// ---------------------------------------------------------------------------
// Rows per lane group, chosen per launch between two instantiations. Measured
// on MI355X (bf16 x; MXFP4 and 3/4/8-bit affine; K from 1536 to 14336, N from
// 1536 to 14336):
//  - B <= 2: one row per lane group is fastest while every wave of the launch
//    fits on the chip at once (256 CUs x 32 waves); beyond that two rows win,
//    as each x slice staged in LDS then serves twice the weight bytes.
//  - 3 <= B <= 7: two rows (four rows cost occupancy: 155+ VGPRs).
//  - B = 8: four rows for MXFP4 and 8-bit affine (MXFP4 K=4096 N=14336: 30.9
//    vs 37.2 us), two for the narrower affine codes (4-bit: 14.2 vs 15.9 us).
template <int NB> constexpr int rows_small() { return 1; }
template <int FMT, int BITS, int NB> constexpr int rows_large() {
    return NB < 8 ? 2 : ((FMT == FMT_AFFINE && BITS < 8) ? 2 : 4);
}
constexpr int64_t kResidentWaves = 256 * 32;
constexpr int kGatherRows = 2;

int ilog2(int v) {
    int r = 0;
    while ((1 << r) < v) ++r;
    return r;
}

// Scale elements per unit, as the formats' glog2 argument: affine
// log2(group / 32); the symmetric block-scaled family log2(block / 32) (-1 for
// blocks of 16); the fixed formats 0.
int scale_glog2(const LaunchParams& p) {
    if (p.format == FMT_AFFINE) return ilog2(p.group / 32);
    if (p.format >= FMT_SB_E8M0) return p.group == 16 ? -1 : ilog2(p.group / 32);
    return 0;
}

// Lanes per row, from K alone, so a row's sum is formed in the same order at
// any N, batch or expert. Rows of at least 64 units: the widest of 64/32/16
// that leaves at most 40% of the lane-unit slots idle. Measured on MI355X,
// spreading a row over more lanes wins even at 62% lane use (8-bit affine,
// K=N=2560: 4.6 us at 64 lanes, 7.4 us at 16). Shorter rows would give each
// lane one partly idle unit and a full cross-lane reduction per unit, so they
// take the widest width that keeps 90% of the slots busy (single calls at
// K=1536 time within 5% across widths; the gathered down projection is 25%
// faster at 16 lanes). Else the least wasteful width.
int pick_lpr(int64_t K) {
    const int64_t U = K >> 5;
    if (U == 0) return 64;
    const double need = U >= 64 ? 0.6 : 0.9;
    int best = 64;
    double best_eff = -1.0;
    for (int lpr : {64, 32, 16}) {
        const int64_t iters = (U + lpr - 1) / lpr;
        const double eff = (double)U / (double)(iters * lpr);
        if (eff >= need) return lpr;
        if (eff > best_eff + 1e-12) { best_eff = eff; best = lpr; }
    }
    return best;
}

// Geometry of a launch staging nb activation rows (and the tile's scales) in
// about `budget` bytes of LDS. The slab length is a multiple of 32 * lpr (or
// all of K), which keeps the lane -> unit map the same for every slab split.
template <int DT, int FMT, int BITS>
Geom make_geom(const LaunchParams& p, int nb, int budget, int rows) {
    using F = Fmt<FMT, BITS>;
    Geom g{};
    g.tiles_per_block = 1;
    g.lpr = pick_lpr(p.K);
    g.lpr_log2 = ilog2(g.lpr);
    g.glog2 = scale_glog2(p);
    g.rows_per_block = kWaves * (64 / g.lpr) * rows;
    const int64_t t = DT == DT_F32 ? 4 : 2;
    const int64_t eb = F::template elem_bytes<DT>();
    const int64_t RB = g.rows_per_block;
    const int64_t U = p.K / 32;
    auto lds_for = [&](int64_t units) {
        const int64_t x = (nb * 32 * units * t + 15) / 16 * 16;
        return x + F::kArrays * RB * F::elem_of_unit(units, g.glog2) * eb;
    };
    int64_t ks_units = U;
    if (U > 0 && lds_for(U) > budget) {
        int64_t nq = budget / lds_for(g.lpr);
        if (nq < 1) nq = 1;
        ks_units = nq * g.lpr < U ? nq * g.lpr : U;
    }
    g.ks = (int)(ks_units > 0 ? 32 * ks_units : 32);
    g.sc_lds_off = (int)((nb * (int64_t)g.ks * t + 15) / 16 * 16);
    // 4-byte copies of the scale rows need every row start, slab start and
    // segment length to be a multiple of 4 bytes
    const int64_t row_stride = p.sc_per_row * eb;
    const int64_t seg_full = F::elem_of_unit(ks_units, g.glog2) * eb;
    const int64_t last_units = ks_units > 0 ? U - ((U - 1) / ks_units) * ks_units : 0;
    const int64_t seg_last = F::elem_of_unit(last_units, g.glog2) * eb;
    bool al = row_stride % 4 == 0 && seg_full % 4 == 0 && seg_last % 4 == 0 &&
              (reinterpret_cast<uintptr_t>(p.scales) & 3) == 0;
    if (F::kArrays == 2) al = al && (reinterpret_cast<uintptr_t>(p.biases) & 3) == 0;
    g.sc_aligned4 = al ? 1 : 0;
    return g;
}

template <int DT, int FMT, int BITS>
size_t stage_bytes(const LaunchParams& p, const Geom& g) {
    using F = Fmt<FMT, BITS>;
    const int64_t units = g.ks / 32;
    return (size_t)g.sc_lds_off + (size_t)(F::kArrays * (int64_t)g.rows_per_block *
                                           F::elem_of_unit(units, g.glog2) *
                                           F::template elem_bytes<DT>());
}

// Dynamic LDS above `free_bytes` (64 KB, less what a kernel holds
// statically) must be requested per kernel and device (gfx950 has 160 KB per
// workgroup). `granted` is the caller's per-instantiation record, per device,
// of the largest size already requested. Requests are made under one lock and
// only ever raise the attribute, so the recorded size is always covered, also
// when threads launch the same kernel with different sizes at once.
constexpr int kMaxDevices = 64;
struct LdsGrant {
    std::atomic<size_t> dev[kMaxDevices];
};
inline std::mutex& lds_grant_mutex() {
    static std::mutex m;
    return m;
}
template <class Kern>
int allow_lds(Kern* kern, size_t bytes, LdsGrant& granted, size_t free_bytes = 64 * 1024) {
    if (bytes <= free_bytes) return 0;
    int d = 0;
    if (const hipError_t e = hipGetDevice(&d); e != hipSuccess) return (int)e;
    if (d < 0 || d >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::atomic<size_t>& slot = granted.dev[d];
    if (bytes <= slot.load(std::memory_order_acquire)) return 0;
    std::lock_guard<std::mutex> lock(lds_grant_mutex());
    if (bytes <= slot.load(std::memory_order_relaxed)) return 0;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)bytes);
    if (e != hipSuccess) return (int)e;
    slot.store(bytes, std::memory_order_release);
    return 0;
}

// Waves a plain QMV launch of R rows per lane group runs.
int64_t launch_waves(const LaunchParams& p, int rows) {
    const int64_t rpb = (int64_t)kWaves * (64 / pick_lpr(p.K)) * rows;
    return (p.N + rpb - 1) / rpb * kWaves;
}

// The short tile applies when K fits one slab, the scale segments are 4-byte
// aligned and a lane holds at most two units of a row.
inline bool short_tile(const LaunchParams& p, const Geom& g) {
    return p.K > 0 && g.ks >= p.K && g.sc_aligned4 && p.K / 32 <= 2 * (int64_t)g.lpr;
}

template <int DT, int FMT, int BITS, int NB, int R>
int launch_qmv_r(const LaunchParams& p, hipStream_t st) {
    const Geom g = make_geom<DT, FMT, BITS>(p, NB, kMaxStageBytes, R);
    const dim3 grid((unsigned)((p.N + g.rows_per_block - 1) / g.rows_per_block));
    const size_t lds = stage_bytes<DT, FMT, BITS>(p, g);
    auto* kern = short_tile(p, g) ? &qmv_kernel<DT, FMT, BITS, NB, R, true>
                                  : &qmv_kernel<DT, FMT, BITS, NB, R, false>;
    static LdsGrant granted_s, granted_l;
    if (const int e = allow_lds(kern, lds, short_tile(p, g) ? granted_s : granted_l)) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, p, g);
    return (int)hipGetLastError();
}

template <int DT, int FMT, int BITS, int NB, int R>
int launch_qmv_norm_r(const LaunchParams& p, const NormArgs& na, hipStream_t st) {
    const Geom g = make_geom<DT, FMT, BITS>(p, NB, kMaxStageBytes, R);
    const dim3 grid((unsigned)((p.N + g.rows_per_block - 1) / g.rows_per_block));
    const size_t lds = stage_bytes<DT, FMT, BITS>(p, g);
    auto* kern = short_tile(p, g) ? &qmv_norm_kernel<DT, FMT, BITS, NB, R, true>
                                  : &qmv_norm_kernel<DT, FMT, BITS, NB, R, false>;
    static LdsGrant granted_s, granted_l;
    if (const int e = allow_lds(kern, lds, short_tile(p, g) ? granted_s : granted_l)) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, p, g, na);
    return (int)hipGetLastError();
}

// The fused RMSNorm + QMV takes four rows per lane group while that still
// launches 2048 waves, else two: every block redoes the row's x work (x *
// gamma and the squares), so fewer, taller blocks do less of it.
template <int DT, int FMT, int BITS>
int launch_qmv_norm_t(const LaunchParams& p, const NormArgs& na, hipStream_t st) {
    switch ((int)p.B) {
#define QMV_CASE(n)                                                                         \
    case n:                                                                                 \
        if (launch_waves(p, 4) >= 2048) return launch_qmv_norm_r<DT, FMT, BITS, n, 4>(p, na, st); \
        return launch_qmv_norm_r<DT, FMT, BITS, n, 2>(p, na, st);
        QMV_CASE(1) QMV_CASE(2) QMV_CASE(3) QMV_CASE(4)
        QMV_CASE(5) QMV_CASE(6) QMV_CASE(7) QMV_CASE(8)
#undef QMV_CASE
        default: return (int)hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// QMV on the matrix cores for several activation rows of the block-scaled
// formats (16-bit activations). With B rows the VALU tile does B dot products
// per decoded code pair, which makes it issue-bound from B = 3 on; here the
// products run on v_mfma_f32_32x32x16 with the weights as the A operand and
// the x rows as the B operand (columns past B repeat row B - 1 and are never
// stored), so the VALU only decodes. A block owns 32 weight rows; its four
// waves take contiguous quarters of the row's 64-code segments, so each wave
// reads whole 128-byte lines over consecutive segments (with segments dealt
// round-robin, four waves shared every line and the kernel fetched most of
// it several times). In a segment a lane (row r = lane % 32, half h = lane / 32) holds
// the 32 codes [32 h, 32 h + 32), one scale block (NVFP4: two), converted in
// registers; k-step s of the MFMA takes codes 32 h + 8 s .. + 8 from both
// operands, so every k slot pairs x and W at the same code. x is staged in
// LDS, zero-padded to whole segments; the four waves' fp32 tiles are added
// in LDS in wave order, then rounded once. The weights load plainly: a line
// is read by four consecutive segment loads of one wave. The sum over a row's K therefore
// runs in a fixed order (per segment inside the MFMA, segments in each wave's
// order, waves 0..3) and every launch gives the same bits.
// ---------------------------------------------------------------------------
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
template <int DT> struct Mfma;
template <> struct Mfma<DT_BF16> {
    typedef __bf16 v8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
    __device__ static inline f32x16_t run(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<DT_F16> {
    typedef _Float16 v8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
    __device__ static inline f32x16_t run(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int kMfmaRows = 32;    // weight rows per block
constexpr int kMfmaDepth = 4;    // segments in flight per lane (a register ring)
constexpr int kMfmaXAhead = 8;   // x chunks per thread loaded ahead of the weights
constexpr int kMfmaRedBytes = kWaves * 32 * 32 * 4;   // the waves' fp32 tiles

// LDS of one launch: x padded to whole 64-code segments, then the waves' tiles
inline size_t mfma_lds_bytes(const LaunchParams& p) {
    const int64_t kpad = (p.K + 63) / 64 * 64;
    return (size_t)(p.B * kpad * 2) + kMfmaRedBytes;
}

template <int DT, int FMT>
__global__ __launch_bounds__(kThreads) void qmv_mfma_kernel(LaunchParams p) {
    static_assert(FMT == FMT_MXFP4 || FMT == FMT_NVFP4 || FMT == FMT_MXFP8, "block-scaled only");
    using S = typename Store<DT>::S;
    using V8 = typename Mfma<DT>::v8;
    constexpr int kCW = FMT == FMT_MXFP8 ? 8 : 4;   // code words per lane and segment
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ln = lane & 31;
    const int hf = lane >> 5;
    const int wave = tid >> 6;
    const int B = (int)p.B;
    const int64_t K = p.K, N = p.N;
    const int kpad = (int)((K + 63) / 64 * 64);
    const int nseg = kpad / 64;
    const int64_t n0 = (int64_t)blockIdx.x * kMfmaRows;
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                     // [B][kpad]
    float* red = reinterpret_cast<float*>(smem + (size_t)B * kpad * 2);   // [kWaves][32 * 32]
    const S* x = static_cast<const S*>(p.x);

    // x chunks: chunk v of the staged [B][kpad] block is row v / (kpad / 8),
    // elements 8 (v % (kpad / 8)) ..; chunks past K are zeros
    const int cpr = kpad / 8;
    const int nchunks = B * cpr;
    auto x_src = [&](int v) __attribute__((always_inline)) {
        const int b = v / cpr;
        const int64_t k = (int64_t)(v - b * cpr) * 8;
        return reinterpret_cast<const v4u*>(x + (int64_t)b * K + (k < K ? k : K - 8));
    };
    auto x_ok = [&](int v) __attribute__((always_inline)) {
        return (int64_t)(v - (v / cpr) * cpr) * 8 < K;
    };
    v4u xa[kMfmaXAhead];
#pragma unroll
    for (int j = 0; j < kMfmaXAhead; ++j) xa[j] = *x_src(min(tid + j * kThreads, nchunks - 1));

    // this lane's weight row (clamped to N - 1) and its segments g = g0 + i,
    // i < cnt: the wave's contiguous quarter of the row
    const int64_t row = n0 + ln < N ? n0 + ln : N - 1;
    const uint8_t* wrow = p.w + row * p.row_bytes;
    const uint8_t* srow = static_cast<const uint8_t*>(p.scales) + row * p.sc_per_row;
    const int per = (nseg + kWaves - 1) / kWaves;
    const int g0 = wave * per;
    const int cnt = nseg > g0 ? (nseg - g0 < per ? nseg - g0 : per) : 0;
    struct Seg {
        uint32_t w[kCW];
        uint32_t s;
    };
    auto load = [&](Seg& b, int i) __attribute__((always_inline)) {
        const int ic = i < cnt ? i : (cnt > 0 ? cnt - 1 : 0);
        const int64_t hk0 = (int64_t)(g0 + ic) * 64 + 32 * hf;
        const int64_t hk = hk0 < K ? hk0 : K - 32;   // first code of the lane's half
        load_words<kCW>(wrow + (FMT == FMT_MXFP8 ? hk : hk / 2), b.w);
        if constexpr (FMT == FMT_NVFP4)   // two E4M3 bytes (the scales may be byte-aligned)
            b.s = (uint32_t)srow[hk / 16] | ((uint32_t)srow[hk / 16 + 1] << 8);
        else
            b.s = srow[hk / 32];
    };
    Seg ring[kMfmaDepth];
    static_for<0, kMfmaDepth>([&](auto d_c) { load(ring[decltype(d_c)::value], decltype(d_c)::value); });

    // x to LDS (the loads above went out before the weights)
#pragma unroll
    for (int j = 0; j < kMfmaXAhead; ++j) {
        const int v = tid + j * kThreads;
        if (v < nchunks)
            *reinterpret_cast<v4u*>(xs + (size_t)v * 8) = x_ok(v) ? xa[j] : v4u{0u, 0u, 0u, 0u};
    }
    for (int v = tid + kMfmaXAhead * kThreads; v < nchunks; v += kThreads)
        *reinterpret_cast<v4u*>(xs + (size_t)v * 8) = x_ok(v) ? *x_src(v) : v4u{0u, 0u, 0u, 0u};
    __syncthreads();

    const uint16_t* xrow = xs + (size_t)(ln < B ? ln : B - 1) * kpad + 32 * hf;
    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    auto step = [&](int i, Seg& b) __attribute__((always_inline)) {
        const int g = g0 + i;
        const bool hv = (int64_t)g * 64 + 32 * hf < K;
        uint32_t a[4][4];
        if constexpr (FMT == FMT_MXFP4) {
            const float sc = __uint_as_float(b.s << 23);
            static_for<0, 4>([&](auto s_c) {
                constexpr int s = decltype(s_c)::value;
                static_for<0, 4>([&](auto e_c) {
                    constexpr int e = decltype(e_c)::value;
                    if constexpr (DT == DT_BF16)
                        a[s][e] = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(b.w[s], sc, e));
                    else
                        a[s][e] = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(b.w[s], sc, e));
                });
            });
        } else if constexpr (FMT == FMT_MXFP8) {
            const float sc = __uint_as_float(b.s << 23);
            static_for<0, 4>([&](auto s_c) {
                constexpr int s = decltype(s_c)::value;
                static_for<0, 2>([&](auto e_c) {
                    constexpr int e = decltype(e_c)::value;
                    const uint32_t wd = b.w[2 * s + e];
                    if constexpr (DT == DT_BF16) {
                        a[s][2 * e] = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd, sc, false));
                        a[s][2 * e + 1] = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd, sc, true));
                    } else {
                        a[s][2 * e] = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wd, sc, false));
                        a[s][2 * e + 1] = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wd, sc, true));
                    }
                });
            });
        } else {
            // E2M1 times its E4M3 block scale, exact in fp32 and in the 16-bit
            // type (at most 6 significant bits); codes 0..15 take the first byte
            const f32x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b.s, 1.0f, false);
            static_for<0, 4>([&](auto s_c) {
                constexpr int s = decltype(s_c)::value;
                const float scs = s < 2 ? sc.x : sc.y;
                static_for<0, 4>([&](auto e_c) {
                    constexpr int e = decltype(e_c)::value;
                    const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b.w[s], 1.0f, e);
                    const f32x2 q = {v.x * scs, v.y * scs};
                    if constexpr (DT == DT_BF16)
                        a[s][e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(q, bf16x2_t));
                    else
                        a[s][e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(q, f16x2_t));
                });
            });
        }
        // a half past K enters as zeros: a select, since the two halves of a
        // wave differ (as a branch it cost a wait for every load in flight)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) a[s][e] = hv ? a[s][e] : 0u;
        load(b, i + kMfmaDepth);
        static_for<0, 4>([&](auto s_c) {
            constexpr int s = decltype(s_c)::value;
            const V8 xb = *reinterpret_cast<const V8*>(xrow + (size_t)g * 64 + 8 * s);
            const V8 wa = __builtin_bit_cast(V8, v4u{a[s][0], a[s][1], a[s][2], a[s][3]});
            acc = Mfma<DT>::run(wa, xb, acc);
        });
    };
    int i = 0;
    for (; i + kMfmaDepth <= cnt; i += kMfmaDepth) {
        static_for<0, kMfmaDepth>([&](auto d_c) {
            constexpr int d = decltype(d_c)::value;
            step(i + d, ring[d]);
        });
    }
    static_for<0, kMfmaDepth>([&](auto d_c) {
        constexpr int d = decltype(d_c)::value;
        if (i + d < cnt) step(i + d, ring[d]);
    });

    // the waves' tiles to LDS (element (m, n): weight row m, activation row n)
    float* mine = red + wave * 32 * 32;
#pragma unroll
    for (int e = 0; e < 16; ++e) mine[(8 * (e >> 2) + 4 * hf + (e & 3)) * 32 + ln] = acc[e];
    __syncthreads();
    const float gmul = (FMT == FMT_NVFP4 && p.gscale) ? *p.gscale : 1.0f;
    for (int idx = tid; idx < 32 * B; idx += kThreads) {
        const int m = idx / B, b = idx - (idx / B) * B;
        if (n0 + m >= N) continue;
        float t = red[m * 32 + b];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) t += red[w * 32 * 32 + m * 32 + b];
        if constexpr (FMT == FMT_NVFP4) t = t * gmul;
        static_cast<S*>(p.y)[(int64_t)b * N + n0 + m] = Store<DT>::from_f32(t);
    }
}

// The matrix-core QMV replaces the VALU tile at B = 8 (bf16 activations,
// MXFP4 / NVFP4 / MXFP8), where the VALU tile does eight dot products per
// decoded pair: K=4096 N=14336 27.6 -> 16.7 us, N=4096 12.2 -> 10.9 us,
// K=1088 N=300 16.6 -> 4.6 us. At B = 3..7 it also wins on some shapes (B=5
// N=14336: 16.5 -> 14.7 us; launches of under 256 VALU waves) but loses on
// others (N=4096: B=4 6.2 vs 9.1 us); it stays at B = 8 so that a row of a
// batch of up to seven equals the same row computed alone, bit for bit (the
// two paths sum in different orders).
constexpr size_t kMfmaMaxLds = 144 * 1024;
inline bool use_mfma_qmv(const LaunchParams& p) {
    return p.B == 8 && p.K > 0 && mfma_lds_bytes(p) <= kMfmaMaxLds;
}

template <int DT, int FMT>
int launch_qmv_mfma(const LaunchParams& p, hipStream_t st) {
    const size_t lds = mfma_lds_bytes(p);
    auto* kern = &qmv_mfma_kernel<DT, FMT>;
    static LdsGrant granted;
    if (const int e = allow_lds(kern, lds, granted)) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)((p.N + kMfmaRows - 1) / kMfmaRows)), dim3(kThreads),
                       lds, st, p);
    return (int)hipGetLastError();
}

template <int DT, int FMT, int BITS>
int launch_qmv_t(const LaunchParams& p, hipStream_t st) {
    if constexpr (DT == DT_BF16 &&
                  (FMT == FMT_MXFP4 || FMT == FMT_NVFP4 || FMT == FMT_MXFP8)) {
        if (use_mfma_qmv(p)) return launch_qmv_mfma<DT, FMT>(p, st);
    }
    const int nb = (int)p.B;
    switch (nb) {
#define QMV_CASE(n)                                                                         \
    case n:                                                                                 \
        if constexpr (n <= 2) {                                                             \
            if (launch_waves(p, rows_small<n>()) <= kResidentWaves)                         \
                return launch_qmv_r<DT, FMT, BITS, n, rows_small<n>()>(p, st);              \
        }                                                                                   \
        return launch_qmv_r<DT, FMT, BITS, n, rows_large<FMT, BITS, n>()>(p, st);
        QMV_CASE(1) QMV_CASE(2) QMV_CASE(3) QMV_CASE(4)
        QMV_CASE(5) QMV_CASE(6) QMV_CASE(7) QMV_CASE(8)
#undef QMV_CASE
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// Blocks a gather launch aims for across the experts that can be active
// (at most min(n_experts, n_slots) of them): about two rounds of resident
// blocks, so each block runs a group of several tiles.
constexpr int64_t kGatherBlocks = 8192;

// Tiles per block of a gather launch: about kGatherBlocks blocks across the
// experts that can be active.
inline int64_t gather_tiles_per_block(const LaunchParams& p, int64_t n_tiles) {
    const int64_t active = p.n_experts < p.n_slots ? p.n_experts : p.n_slots;
    int64_t tpb = (n_tiles * active + kGatherBlocks - 1) / kGatherBlocks;
    if (tpb < 1) tpb = 1;
    if (tpb > n_tiles) tpb = n_tiles > 0 ? n_tiles : 1;
    return tpb;
}

template <int DT, int FMT, int BITS>
int launch_gather_t(const LaunchParams& p, hipStream_t st) {
    const NoMoeArgs none{};
    constexpr int kChunk = gather_chunk_for(DT);
    Geom g = make_geom<DT, FMT, BITS>(p, kChunk, kGatherStageBytes, kGatherRows);
    g.out_rows = g.rows_per_block;
    const int64_t n_tiles = (p.N + g.out_rows - 1) / g.out_rows;
    const int64_t tpb = gather_tiles_per_block(p, n_tiles);
    g.tiles_per_block = (int)tpb;
    const dim3 grid((unsigned)((n_tiles + tpb - 1) / tpb), (unsigned)(p.n_experts + 1));
    const size_t lds = stage_bytes<DT, FMT, BITS>(p, g);
    if (g.ks >= p.K && p.K > 0)
        hipLaunchKernelGGL((gather_kernel<DT, FMT, BITS, kGatherRows, true>), grid,
                           dim3(kThreads), lds, st, p, g, none);
    else
        hipLaunchKernelGGL((gather_kernel<DT, FMT, BITS, kGatherRows, false>), grid,
                           dim3(kThreads), lds, st, p, g, none);
    return (int)hipGetLastError();
}

// Fused gate/up + activation: the gather over slots s = t * top_k + j with
// each lane group producing one output row from its gate and up rows. Needs
// the chunk's x rows for all of K in LDS (up to 64 KB).
template <int DT, int FMT, int BITS>
int launch_moe_gate_up_t(const LaunchParams& p, const MoeArgs& m, hipStream_t st) {
    constexpr int kChunk = gather_chunk_for(DT);
    // one slab of all of K; the pipelined loop reads its scales from global
    // memory, so LDS holds just the chunk's x rows
    Geom g = make_geom<DT, FMT, BITS>(p, kChunk, 1 << 30, kGatherRows);
    const size_t lds = (size_t)kChunk * (size_t)p.K * (DT == DT_F32 ? 4 : 2);
    if (g.ks < p.K || p.K <= 0 || lds > (size_t)kMaxStageBytes) return (int)hipErrorInvalidValue;
    g.out_rows = g.rows_per_block / kGatherRows;
    const int64_t n_tiles = (p.N + g.out_rows - 1) / g.out_rows;
    const int64_t tpb = gather_tiles_per_block(p, n_tiles);
    g.tiles_per_block = (int)tpb;
    const dim3 grid((unsigned)((n_tiles + tpb - 1) / tpb), (unsigned)(p.n_experts + 1));
    auto* kern = &gather_kernel<DT, FMT, BITS, kGatherRows, true, kGatherSwiglu>;
    // the static slot lists ride on top of the dynamic x stage
    static LdsGrant granted;
    if (const int e = allow_lds(kern, lds, granted, 32 * 1024)) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, p, g, m);
    return (int)hipGetLastError();
}

// Down projection summed over each token's slots: all of K for up to top_k
// mid rows in LDS (at most 64 KB).
template <int DT, int FMT, int BITS>
int launch_moe_down_t(const LaunchParams& p, const MoeArgs& m, hipStream_t st) {
    constexpr int R = kGatherRows;
    const int64_t tb = DT == DT_F32 ? 4 : 2;
    const size_t lds = (size_t)(m.top_k * p.K * tb);
    if (m.top_k > kMaxTopK || lds > (size_t)kMaxStageBytes) return (int)hipErrorInvalidValue;
    Geom g{};
    g.lpr = pick_lpr(p.K);
    g.lpr_log2 = ilog2(g.lpr);
    g.glog2 = scale_glog2(p);
    g.rows_per_block = kWaves * (64 / g.lpr) * R;
    g.out_rows = g.rows_per_block;
    g.ks = (int)p.K;
    const int64_t n_tiles = (p.N + g.out_rows - 1) / g.out_rows;
    int64_t tpb = (n_tiles * p.n_x_rows + kGatherBlocks - 1) / kGatherBlocks;
    if (tpb < 1) tpb = 1;
    if (tpb > n_tiles) tpb = n_tiles;
    g.tiles_per_block = (int)tpb;
    const dim3 grid((unsigned)((n_tiles + tpb - 1) / tpb), (unsigned)p.n_x_rows);
    auto* kern = &moe_down_kernel<DT, FMT, BITS, R>;
    static LdsGrant granted;
    if (const int e = allow_lds(kern, lds, granted, 32 * 1024)) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, p, g, m);
    return (int)hipGetLastError();
}

template <int DT, int FMT, int BITS>
int launch_dequant_t(const LaunchParams& p, float* out, hipStream_t st) {
    const int64_t n = p.N * (p.K >> 5);
    const int glog2 = scale_glog2(p);
    hipLaunchKernelGGL((dequant_kernel<DT, FMT, BITS>), dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, st, p, glog2, out);
    return (int)hipGetLastError();
}

}  // namespace
}  // namespace qmv
