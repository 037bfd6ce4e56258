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
// exactly once, by one thread); staged() runs in every thread after the
// last of its elements has been staged and before the barrier that publishes
// them, settled() in every thread right after that barrier; out(b, v) is row
// b's fp32 result before the final rounding.
template <class S> struct XContig {
    using Chunk = v4u;
    const S* x;
    int64_t K;
    __device__ const S* row(int b) const { return x + (int64_t)b * K; }
    __device__ Chunk load(int b, int64_t k) const {
        return *reinterpret_cast<const v4u*>(row(b) + k);
    }
    __device__ v4u stage(int, int64_t, const Chunk& c) const { return c; }
    __device__ void staged() const {}
    __device__ void settled() const {}
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
    __device__ void staged() const {}
    __device__ void settled() const {}
    __device__ float out(int, float v) const { return v; }
};
// Fused RMSNorm. The row's normalization r[b] = 1 / sqrt(mean_k x^2 + eps) is
// one scalar, so it multiplies the fp32 dot products at the end; element k
// enters LDS as RN_T(x[b, k] * gamma[k]) — the product of two T values is
// exact in fp32, so that is one rounding of the exact product. The squares
// are summed as the elements are staged (fp32, each thread in its staging
// order), then over the lanes of each wave (staged(), before the barrier that
// publishes the staged x) and over the waves in a fixed order (settled(),
// after it), so every block of a launch forms the same r, and r is known
// before the first weight unit is folded: the block needs no barrier of its
// own for it.
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
    // the wave's sum by DPP lane moves (VALU latency, no LDS round trips on
    // the way to the barrier), left in lane 63
    __device__ void staged() const {
        const int lane = threadIdx.x & 63;
        const int wave = threadIdx.x >> 6;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float t = group_sum(ss[b], 64);
            if (lane == 63) red[b * kWaves + wave] = t;
        }
    }
    __device__ void settled() const {
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

// Block index -> row-tile index of the QMV kernels. Consecutive blocks go
// to the eight XCDs in turn, so with the identity map every 64 consecutive
// rows (one 128-byte line of a 16-bit y) were computed and written by all
// eight XCDs. Here each group of 64 blocks is reordered so that the eight
// blocks an XCD receives from it own eight consecutive row tiles: an XCD
// reads 64 consecutive weight rows and writes whole lines of y. Blocks past
// the last whole group keep their index. Measured on the MXFP4 K=4096
// N=14336 row kernel with groups of 2, 4, 8, 16, 32 and 224 blocks per XCD:
// 6.65, 6.63, 6.59, 6.61, 6.62, 6.62 us against 6.77 us for the identity.
__device__ inline int64_t xcd_chunked_block(int64_t b, int64_t grid) {
    constexpr int64_t kXcds = 8, kPerXcd = 8, kSpan = kXcds * kPerXcd;
    if (b >= (grid / kSpan) * kSpan) return b;
    const int64_t r = b % kSpan;
    return (b - r) + (r % kXcds) * kPerXcd + r / kXcds;
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
        const bool last = kShort || slab + ks >= K;
        if (last) xr.staged();
        __syncthreads();
        if (last) xr.settled();

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
        // LDS is restaged for the next slab, or by the caller's next tile
        // (the gather); a one-slab tile of the QMV kernels ends here
        if constexpr (!kShort) __syncthreads();
    }

    // reduce over the LPR lanes of each row group (result in its last lane)
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            total[i][b] = group_sum(total[i][b], lpr);
        }

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
    qmv_tile<DT, FMT, BITS, NB, R, true, SHORT>(p, g,
                                                xcd_chunked_block(blockIdx.x, gridDim.x) *
                                                    g.rows_per_block,
                                                p.w, p.scales, p.biases, xr, yrow, gmul, lds);
}

// ---------------------------------------------------------------------------
// One to four activation rows of 16-bit values (NB) against MXFP4 / NVFP4 /
// MXFP8 weights or 4-bit affine codes with K = 2048 * NU: the tile above cut
// to what this case needs. The block stages its NB x rows in LDS, each in the layout the tile
// gives one row, and every unit is folded against all of them. Each wave
// takes two rows (its row index is wave-uniform, so row addresses live in
// scalar registers); lane l takes units l, l + 64, ... of both rows, exactly
// the units and the order of the tile with 64 lanes per row, and folds them
// with the tile's unit_fma against x staged in LDS in the tile's layout. The
// scale bytes of a lane's units are loaded by the lane itself (64 lanes read
// 64 consecutive scale elements of a row) instead of being staged, and no
// clamped or predicated index is formed per lane. A
// row's result is therefore the tile's bit for bit; the saving is the
// staging and addressing work (VALU), which at one activation row is most of
// what the tile does besides the decode and the dot products.
// ---------------------------------------------------------------------------
template <int FMT> constexpr int row_units_max() { return 2; }


template <int DT, int FMT, int BITS, int NU, class XR, int NB = 1, int R = 2>
__device__ inline void row_tiles(const LaunchParams& p, const XR& xr, float gmul,
                                 typename Store<DT>::S* xs) {
    using F = Fmt<FMT, BITS>;
    using S = typename Store<DT>::S;
    constexpr int W = F::kWords;
    constexpr int kUnitBytes = 4 * W;
    constexpr int KR = 2048 * NU;             // elements per row
    constexpr int US = KR / 32;               // units per row
    // x sits in LDS in the tile's four planes (plane SC holds the 16-byte
    // piece SC of every unit), each plane padded by 64 bytes so that the 16
    // lanes of a staging write (4 units x 4 planes) hit all 64 banks once;
    // unit_fma takes the plane stride in units
    constexpr int USP = US + 4;
    constexpr int XS = 32 * USP;              // LDS elements per staged x row
    constexpr int kEB = F::template elem_bytes<DT>();

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t N = p.N;
    const int64_t row0 = xcd_chunked_block(blockIdx.x, gridDim.x) * (kWaves * R) + wave * R;

    // (1) this thread's NU 16-byte chunks of x (and whatever the accessor's
    // staging reads with them), ahead of the weights
    typename XR::Chunk xc[NB][NU];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < NU; ++j) xc[b][j] = xr.load(b, (int64_t)(tid + j * kThreads) * 8);

    // (2) the lane's units of both rows and their scale elements (rows past
    // the end re-read row N - 1; their results are not stored)
    UnitRaw<FMT, BITS, R> u_raw[NU];
    typename F::Raw s_raw[NU][R];
    // affine: units per scale group, log2 (groups of 32, 64 or 128 codes)
    const int glog2 = FMT == FMT_AFFINE ? 31 - __builtin_clz((unsigned)p.group >> 5) : 0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t r = row0 + i < N ? row0 + i : N - 1;
        const uint8_t* wrow = p.w + r * p.row_bytes;
        const uint8_t* srow = static_cast<const uint8_t*>(p.scales) + r * p.sc_per_row * kEB;
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            load_words<W, true>(wrow + (lane + 64 * j) * kUnitBytes, u_raw[j].d[i]);
            // the unit's scale elements (one E8M0 byte, NVFP4's two E4M3
            // bytes, nontemporal like the weights; or its group's affine
            // scale and bias)
            if constexpr (FMT == FMT_AFFINE)
                s_raw[j][i] = F::template global_raw<DT>(
                    static_cast<const uint8_t*>(p.scales), static_cast<const uint8_t*>(p.biases),
                    (uint32_t)(r * p.sc_per_row * kEB), lane + 64 * j, glog2);
            else if constexpr (FMT == FMT_NVFP4)
                s_raw[j][i].e = __builtin_nontemporal_load(
                    reinterpret_cast<const uint16_t*>(srow) + (lane + 64 * j));
            else
                s_raw[j][i].e = __builtin_nontemporal_load(srow + (lane + 64 * j));
        }
    }

    // (3) x to LDS, chunk v at the tile's slot, in the tile's staging order
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const int v = tid + j * kThreads;
            *reinterpret_cast<v4u*>(xs + b * XS + x_lds_slot(v * 8, USP)) =
                stage_vec<FMT, BITS, DT>(xr.stage(b, (int64_t)v * 8, xc[b][j]));
        }
    xr.staged();
    __syncthreads();
    xr.settled();

    // (4) the units in the tile's order, (5) the tile's reduction and store
    float total[R][NB];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) total[i][b] = 0.0f;
#pragma unroll
    for (int j = 0; j < NU; ++j) {
        typename F::Scale scl[R];
#pragma unroll
        for (int i = 0; i < R; ++i) scl[i] = F::template decode<DT>(s_raw[j][i]);
        unit_fma<DT, FMT, BITS, NB, R>(u_raw[j], scl, xs, lane + 64 * j, XS, USP, total);
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) total[i][b] = group_sum(total[i][b], 64);
    if (lane == 63) {
        S* y = static_cast<S*>(p.y);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            if (row0 + i < N) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    float v = xr.out(b, total[i][b]);
                    if constexpr (FMT == FMT_NVFP4) v = v * gmul;
                    y[b * N + row0 + i] = Store<DT>::from_f32(v);
                }
            }
        }
    }
}

template <int DT, int FMT, int BITS, int NU, int NB = 1, int R = 2>
__global__ __launch_bounds__(kThreads) void qmv_row_kernel(LaunchParams p) {
    using S = typename Store<DT>::S;
    __shared__ __align__(16) S xs[NB * (2048 * NU / 32 + 4) * 32];
    const XContig<S> xr{static_cast<const S*>(p.x), p.K};
    const float gmul = (FMT == FMT_NVFP4 && p.gscale) ? *p.gscale : 1.0f;
    row_tiles<DT, FMT, BITS, NU, XContig<S>, NB, R>(p, xr, gmul, xs);
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
    qmv_tile<DT, FMT, BITS, NB, R, true, SHORT>(p, g,
                                                xcd_chunked_block(blockIdx.x, gridDim.x) *
                                                    g.rows_per_block,
                                                p.w, p.scales, p.biases, xr, yrow, gmul, lds);
}

// The fused RMSNorm + QMV at one activation row on the one-row kernel's
// structure (16-bit activations, MXFP4 / NVFP4 / MXFP8, K = 2048 or 4096):
// the XNorm accessor stages x times gamma with the tile's chunk-to-thread
// assignment and sums the squares in the same order, so r and every result
// are bit for bit those of qmv_norm_kernel.
template <int DT, int FMT, int BITS, int NU, int NB = 1>
__global__ __launch_bounds__(kThreads) void qmv_row_norm_kernel(LaunchParams p, NormArgs na) {
    using S = typename Store<DT>::S;
    __shared__ __align__(16) S xs[NB * (2048 * NU / 32 + 4) * 32];
    __shared__ float red[NB * kWaves];
    const XNorm<DT, NB> xr{static_cast<const S*>(p.x), p.K, static_cast<const S*>(na.gamma),
                           na.eps, red, {}, {}};
    const float gmul = (FMT == FMT_NVFP4 && p.gscale) ? *p.gscale : 1.0f;
    row_tiles<DT, FMT, BITS, NU, XNorm<DT, NB>, NB, 2>(p, xr, gmul, xs);
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
constexpr int kGatherChunkMax = 4;
__host__ __device__ constexpr int gather_chunk_for(int dt) { return dt == DT_F32 ? 2 : kGatherChunkMax; }
constexpr int kGatherStageBytes = 40 * 1024;

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

// The gather tile loop for 16-bit activations and MXFP4 / NVFP4 / MXFP8
// weights with K = 2048 * NU (one slab, 64 lanes per row): the one-row QMV
// kernel's structure applied to the gather's tiles. Each wave owns the same
// two rows of every tile of its group (plain mode: rows 2 w, 2 w + 1; pair
// mode: output row w, its gate row from w and its up row from w2), with the
// row addresses wave-uniform; lane l takes units l, l + 64, ... of both rows,
// exactly the units and the order of gather_tiles, folded by the same
// unit_fma and reduced by the same group_sum, so every result is bit for bit
// that of gather_tiles. The next tile's weight and scale loads are issued
// before the current tile is folded. What it removes is the generic loop's
// per-unit bookkeeping (cursor, tile entry, per-lane offsets and clamps),
// which at a few slots per expert is much of its VALU work.
// Variants of the lean gather loop (a kernel template argument, 0 = the
// generic loop): 1 and 2 take 64 lanes per row and K = 2048 or 4096; 3 takes
// 16 lanes per row and K = 1536 (three units per lane).
__host__ __device__ constexpr int row_lpr(int nur) { return nur == 3 ? 16 : 64; }
__host__ __device__ constexpr int row_nu(int nur) { return nur; }

template <int DT, int FMT, int BITS, int NB, int NU, int LPR, int MODE = kGatherPlain>
__device__ inline void gather_row_tiles(const LaunchParams& p, const MoeArgsOf<MODE>& m,
                                        const Geom& g, int64_t tile0, int64_t tile_end,
                                        const uint8_t* __restrict__ w, const void* sc,
                                        const void* bi,
                                        typename Store<DT>::S* const (&yrow)[NB], float gmul,
                                        const typename Store<DT>::S* lds) {
    using F = Fmt<FMT, BITS>;
    constexpr int R = 2;
    constexpr int W = F::kWords;
    constexpr int kUnitBytes = 4 * W;
    constexpr int US = LPR * NU;              // units per row
    constexpr int KR = 32 * US;
    constexpr int kGroups = 64 / LPR;         // lane groups (row pairs) per wave
    constexpr bool kPair = MODE == kGatherSwiglu;
    struct Item {
        UnitRaw<FMT, BITS, R> u[NU];
        typename F::Raw raw[NU][R];
    };
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane / LPR;               // this lane's row pair within the wave
    const int gl = lane % LPR;
    const int slot = wave * kGroups + grp;    // row pair (plain) or output row (pair) index
    const int64_t N = p.N;
    const int64_t RB = g.out_rows;
    const int64_t sc_row_bytes = p.sc_per_row * F::template elem_bytes<DT>();
    const uint8_t* w_of[2] = {w, w};
    const uint8_t* sc_of[2] = {static_cast<const uint8_t*>(sc), static_cast<const uint8_t*>(sc)};
    const uint8_t* bi_of[2] = {static_cast<const uint8_t*>(bi), static_cast<const uint8_t*>(bi)};
    if constexpr (kPair) {
        w_of[1] = m.w2;
        sc_of[1] = static_cast<const uint8_t*>(m.scales2);
        bi_of[1] = static_cast<const uint8_t*>(m.biases2);
    }
    // row of operand row i in tile t (rows past N re-read row N - 1)
    auto row_of = [&](int64_t t, int i) __attribute__((always_inline)) {
        const int64_t r = kPair ? t * RB + slot : t * RB + R * slot + i;
        return r < N ? r : N - 1;
    };
    auto load = [&](Item& it, int64_t t) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t r = row_of(t, i);
            const int mi = kPair ? i : 0;
            const uint8_t* wr = w_of[mi] + r * p.row_bytes;
            // (an expert's scale arrays hold at most N x 256 bytes: 32-bit offsets)
            const uint32_t so = (uint32_t)(r * sc_row_bytes);
#pragma unroll
            for (int j = 0; j < NU; ++j) {
                load_words<W>(wr + (gl + LPR * j) * kUnitBytes, it.u[j].d[i]);
                it.raw[j][i] = F::template global_raw<DT>(sc_of[mi], bi_of[mi], so, gl + LPR * j,
                                                          g.glog2);
            }
        }
    };
    auto fold_store = [&](const Item& it, int64_t t) __attribute__((always_inline)) {
        float total[R][NB];
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int b = 0; b < NB; ++b) total[i][b] = 0.0f;
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            typename F::Scale scl[R];
#pragma unroll
            for (int i = 0; i < R; ++i) scl[i] = F::template decode<DT>(it.raw[j][i]);
            unit_fma<DT, FMT, BITS, NB, R>(it.u[j], scl, lds, gl + LPR * j, KR, US, total);
            // keep each unit's LDS reads next to their use (hoisting them all
            // ahead of the arithmetic doubles the register footprint)
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int b = 0; b < NB; ++b) total[i][b] = group_sum(total[i][b], LPR);
        if (gl == LPR - 1) {
            if constexpr (kPair) {
                const int64_t r = t * RB + slot;
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
                    const int64_t r = t * RB + R * slot + i;
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
    };
    // two tiles in flight: fold one while the next one's loads are out
    Item a, b;
    int64_t t = tile0;
    load(a, t);
    for (; t + 1 < tile_end; t += 2) {
        load(b, t + 1);
        fold_store(a, t);
        if (t + 2 < tile_end) load(a, t + 2);
        fold_store(b, t + 1);
    }
    if (t < tile_end) fold_store(a, t);
}

template <int DT, int FMT, int BITS, int R, bool kOneSlab, int MODE, int NUR = 0>
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
            if constexpr (NUR > 0)
                gather_row_tiles<DT, FMT, BITS, NB, row_nu(NUR), row_lpr(NUR), MODE>(
                    p, m, g, tile0, tile_end, w, sc, bi, yrow, gmul, lds);
            else
                gather_tiles<DT, FMT, BITS, NB, R, MODE>(p, m, g, tile0, tile_end, w, sc, bi,
                                                         yrow, gmul, lds);
        } else {
            static_assert(MODE == kGatherPlain, "the paired mode needs one slab");
            for (int64_t t = tile0; t < tile_end; ++t)
                qmv_tile<DT, FMT, BITS, NB, R>(p, g, t * RB, w, sc, bi, xr, yrow, gmul,
                                               lds);
        }
    };
    if constexpr (gather_chunk_for(DT) > 2) {
        switch (cnt) {
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            default: run(std::integral_constant<int, 4>{}); break;
        }
    } else {
        if (cnt == 1)
            run(std::integral_constant<int, 1>{});
        else
            run(std::integral_constant<int, 2>{});
    }
}

// kOneSlab: K > 0 and the geometry holds all of K in one slab (the launcher
// checks), so the group runs gather_tiles; otherwise qmv_tile per tile.
// MODE kGatherSwiglu: the fused gate/up projection of the routed-MoE block
// (slot s reads x row s / top_k; w / w2 are the gate / up matrices; the output
// is the activation, one row per slot).
template <int DT, int FMT, int BITS, int R, bool kOneSlab, int MODE = kGatherPlain, int NUR = 0>
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
        gather_chunk<DT, FMT, BITS, R, kOneSlab, MODE, NUR>(p, m, g, tile0, tile_end, w, sc, bi,
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

template <int FMT> inline bool use_mfma_qmv(const LaunchParams& p);
template <int FMT> inline bool use_mfma_norm_f16(const LaunchParams& p);
template <int DT, int FMT, bool NORM>
int launch_qmv_mfma(const LaunchParams& p, const NormArgs& na, hipStream_t st);

// Activation rows the one-row kernel takes (it folds each row exactly as a
// one-row call does, so every batch row equals that call bit for bit). Picked
// from measurements at K=4096, N=14336 against the matrix cores (bf16) and the
// VALU tile (f16), in one process (row kernel / the path it replaced, us):
//   bf16 MXFP4  B=2 7.68 / 8.68    B=3 8.95 / 8.73 (matrix cores kept)
//   bf16 NVFP4  B=2 7.89 / 8.70    B=3 9.21 / 10.74   B=4 11.35 / 10.81 (kept)
//   bf16 MXFP8  B=2 12.22 / 12.32  B=3 12.82 / 13.65  B=4 13.95 / 15.67
// Two weight rows per wave at every batch size (four rows per wave at B=3 and
// B=4 ran 9-15 % slower: half the waves, each with twice the loads and decode
// before its first product).
// The one-row kernel's instances: 16-bit x with the MX formats or 4-bit affine
// codes (each lane loads its units' scale and bias elements; x is staged in
// the packed path's pair order). 4-bit affine g64 at K = N = 4096 against the
// VALU tile (us, tile / one-row kernel, one process): bf16 B=1 4.62 / 4.00,
// B=2 5.38 / 4.78, B=3 6.24 / 5.39, B=4 7.03 / 6.10; f16 B=1 4.43 / 3.98, B=4
// 6.63 / 5.67; the fused RMSNorm bf16 B=1 5.19 / 4.60, B=4 9.55 / 8.63.
template <int DT, int FMT, int BITS> constexpr bool row_kernel_ok() {
    return DT != DT_F32 && (FMT == FMT_MXFP4 || FMT == FMT_NVFP4 || FMT == FMT_MXFP8 ||
                            (FMT == FMT_AFFINE && BITS == 4));
}
template <int DT, int FMT> constexpr int row_max_batch() {
    if constexpr (FMT == FMT_AFFINE) return 4;
    if constexpr (DT == DT_BF16) return FMT == FMT_MXFP4 ? 2 : FMT == FMT_NVFP4 ? 3 : 4;
    return 4;
}
// Activation rows the fused RMSNorm's one-row kernel takes (each batch row
// equals its one-row call bit for bit, its r included): the plain kernel's
// limits, which the same measurement gave (K=4096, N=14336, one process; us,
// row kernel / the path it replaced):
//   bf16 MXFP4  B=2 10.22 / 11.17  B=3 12.73 / 11.10 (matrix cores kept)
//   bf16 NVFP4  B=2 10.33 / 13.07  B=3 13.15 / 16.68  B=4 15.92 / 15.45 (kept)
//   bf16 MXFP8  B=2 13.69 / 15.11  B=3 16.15 / 18.96  B=4 17.92 / 19.51
//   f16 (VALU tile replaced) MXFP4 B=4 15.61 / 15.67, NVFP4 16.36 / 18.16,
//   MXFP8 18.01 / 19.93, and B = 2, 3 gain 2-21 %.
template <int DT, int FMT> constexpr int row_norm_max_batch() { return row_max_batch<DT, FMT>(); }
template <int DT, int FMT, int BITS, int NU, int NB>
int launch_row_norm(const LaunchParams& p, const NormArgs& na, hipStream_t st) {
    const dim3 grid((unsigned)((p.N + 2 * kWaves - 1) / (2 * kWaves)));
    hipLaunchKernelGGL((qmv_row_norm_kernel<DT, FMT, BITS, NU, NB>), grid, dim3(kThreads), 0, st,
                       p, na);
    return (int)hipGetLastError();
}
template <int DT, int FMT, int BITS, int NU>
int launch_row_norm_nu(const LaunchParams& p, const NormArgs& na, hipStream_t st) {
    constexpr int kMax = row_norm_max_batch<DT, FMT>();
    switch ((int)p.B) {
        case 2: if constexpr (kMax >= 2) return launch_row_norm<DT, FMT, BITS, NU, 2>(p, na, st); break;
        case 3: if constexpr (kMax >= 3) return launch_row_norm<DT, FMT, BITS, NU, 3>(p, na, st); break;
        case 4: if constexpr (kMax >= 4) return launch_row_norm<DT, FMT, BITS, NU, 4>(p, na, st); break;
        default: break;
    }
    return launch_row_norm<DT, FMT, BITS, NU, 1>(p, na, st);
}

// The fused RMSNorm + QMV takes the one-row kernel and the matrix cores where
// the plain QMV does (16-bit batches of the MX formats at K = 2048 / 4096 up
// to row_norm_max_batch rows; bf16 batches from mf_min_batch rows otherwise);
// on the VALU tile it takes four rows per lane group while that still launches
// 2048 waves, else two: every block redoes the row's x work (x * gamma and the
// squares), so fewer, taller blocks do less of it.
template <int DT, int FMT, int BITS>
int launch_qmv_norm_t(const LaunchParams& p, const NormArgs& na, hipStream_t st) {
    if constexpr (row_kernel_ok<DT, FMT, BITS>()) {
        if (p.B <= row_norm_max_batch<DT, FMT>() && p.N > 0 && p.K > 0 && p.K % 2048 == 0 &&
            p.K / 2048 <= row_units_max<FMT>()) {
            if (p.K == 2048) return launch_row_norm_nu<DT, FMT, BITS, 1>(p, na, st);
            return launch_row_norm_nu<DT, FMT, BITS, 2>(p, na, st);
        }
    }
    if constexpr (DT == DT_BF16 &&
                  (FMT == FMT_MXFP4 || FMT == FMT_NVFP4 || FMT == FMT_MXFP8)) {
        if (use_mfma_qmv<FMT>(p)) return launch_qmv_mfma<DT, FMT, true>(p, na, st);
    }
    if constexpr (DT == DT_F16 &&
                  (FMT == FMT_MXFP4 || FMT == FMT_NVFP4 || FMT == FMT_MXFP8)) {
        if (use_mfma_norm_f16<FMT>(p)) return launch_qmv_mfma<DT, FMT, true>(p, na, st);
    }
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
// QMV on the matrix cores for 3..8 activation rows of the block-scaled
// formats (bf16 activations). With B rows the VALU tile does B dot products
// per decoded code pair, which makes it issue-bound from B = 3 on; here the
// products run on v_mfma_f32_16x16x32_bf16 with the weights as the A operand
// (16 weight rows) and the activation rows as the B operand columns (16
// columns, of which B are used), so the VALU only decodes.
//
// A block owns RT 16-row tiles of weight rows (mf_tiles: four for MXFP4, two
// otherwise) and all of K; its W waves take chunks of 128 weight bytes per
// row (256 FP4 or 128 FP8 codes), chunk c going to wave c mod W, and a wave's
// activation pieces serve all its tiles. A chunk is loaded with 2 RT
// coalesced loads (lane l
// reads 16 bytes of row 8 i + l / 8, so eight consecutive lanes cover one
// 128-byte line), written to the wave's own LDS area and read back in the
// MFMA operand layout: lane 16 q + r holds the 32 codes [32 q, 32 q + 32) of
// a 128-code segment of row r, one MX scale block, and MFMA t of the segment
// takes codes 8 t .. 8 t + 7 of every lane's 32 (the same k order in A and
// B). The 16-byte pieces are stored XOR-swizzled by row so the operand reads
// hit distinct LDS banks. x values enter the B operand straight from global
// memory (lanes of column b < B), loaded together with the chunk's weights.
// When K is a whole number of chunks and the scale rows are short, the
// block's scale rows are staged in LDS once (behind one barrier that the
// first chunk's loads are already in flight across) and each chunk reads its
// scale bytes from there; otherwise each lane gathers its scale bytes from
// global memory. Codes at k >= K enter as zeros, together with their x values.
//
// Each output is one MFMA accumulator element per wave, summed over that
// wave's chunks in order; the W partial sums are added in wave order in LDS
// and rounded once. A row's result depends on K and its own data only, and a
// column's on its own x row only, so tail rows equal a padded call and every
// activation row equals the same row in any other batch of 3..8 rows, bit
// for bit.
// ---------------------------------------------------------------------------
template <int DT> struct Mfma16;
template <> struct Mfma16<DT_BF16> {
    typedef __bf16 v8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
};
typedef float mf_f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));

// Raw (unswizzled) buffer resources: the fourth descriptor word of gfx9
// targets (32-bit data format), and an offset past every buffer this file
// builds one for (such buffers hold fewer bytes; loads there return zeros).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kBufferOutOfRange = 0x7FFFFF00;

constexpr int kMfChunkBytes = 128;   // weight bytes per row and chunk
constexpr int kMfMaxScaleRow = 256;  // scale bytes per row the staged path takes

// codes per chunk and 128-code segments per chunk
template <int FMT> constexpr int mf_chunk_codes() { return FMT == FMT_MXFP8 ? 128 : 256; }

// 16-row tiles per block and waves per block (one per chunk, at most this
// many; each wave stages 2 KB per tile of its chunk in LDS). MXFP4 takes four
// tiles and eight waves: every wave's activation pieces then serve 64 rows,
// which halves the x bytes the launch moves from L2 (at B = 8 as many as the
// weights) and measured 12.4 -> 10.8 us at B = 8 (K=4096, N=14336; 48-, 80-
// and 128-row blocks and four waves were slower). NVFP4 and MXFP8, whose
// decode is heavier and whose waves then run twice the work per chunk in
// turn, measured slower that way (19.3 and 25.2 us against 12.6 and 20.2)
// and keep two tiles: eight waves for NVFP4 (fp32 products, 88 VGPRs), 16
// for MXFP8, 8 for the general instances (82..108 VGPRs).
// The fused-RMSNorm form of NVFP4 takes four tiles as well: its x * gamma
// work per chunk is then shared by twice the rows (K=4096 N=14336, B = 4 / 8:
// 19.2 / 19.5 -> 15.4 / 15.4 us; the plain NVFP4 QMV with four tiles ran
// 12.0 / 12.3 against 10.8 / 11.6 us).
template <int FMT, bool kWhole, bool NORM = false> constexpr int mf_tiles() {
    return (kWhole && (FMT == FMT_MXFP4 || (NORM && FMT == FMT_NVFP4))) ? 4 : 2;
}
template <int FMT, bool kWhole> constexpr int mf_max_waves() {
    return (kWhole && FMT == FMT_MXFP8) ? 16 : 8;
}
// 16-byte scale pieces each thread stages (kWhole): a block's scale rows,
// at most kMfMaxScaleRow bytes each, over at least 64 threads per wave of the
// launch (the launcher checks that they fit)
template <int FMT, bool kWhole, bool NORM = false> constexpr int mf_scale_pieces() {
    constexpr int per = 16 * mf_tiles<FMT, kWhole, NORM>() * kMfMaxScaleRow / 16;
    constexpr int thr = 64 * mf_max_waves<FMT, kWhole>();
    return kWhole ? (per + thr - 1) / thr : 1;
}
inline int mfma_waves(const LaunchParams& p, int max_waves) {
    const int cc = p.format == FMT_MXFP8 ? 128 : 256;
    const int64_t chunks = (p.K + cc - 1) / cc;
    return (int)(chunks < max_waves ? (chunks > 0 ? chunks : 1) : max_waves);
}

// kWhole: K is a multiple of the chunk and the scale rows allow vector loads
// (every chunk is whole); otherwise codes past K are zeroed by selects and
// the scale bytes are loaded one by one.
//
// NORM: the fused RMSNorm in front (y[b] = r[b] * (W . RN_T(x[b] * gamma)),
// r[b] = 1 / sqrt(mean_k x[b, k]^2 + eps)). Each x piece is loaded with the
// matching gamma piece and enters the B operand as RN_T(x * gamma) (one
// rounding of the exact product, as the VALU tile stages it); each lane sums
// the squares of its x values (fp32, in its chunk and piece order), and the
// block adds the lanes' sums over the four lane quarters and the waves in a
// fixed order with the partial tiles, so every block forms the same r[b],
// which multiplies the row's sum before the NVFP4 global scale.
template <int DT, int FMT, bool kWhole, bool NORM>
__device__ inline void mfma_tile(const LaunchParams& p, const NormArgs& na) {
    static_assert(FMT == FMT_MXFP4 || FMT == FMT_NVFP4 || FMT == FMT_MXFP8, "block-scaled only");
    using S = typename Store<DT>::S;
    using V8 = typename Mfma16<DT_BF16>::v8;
    // f16 activations: column c < 8 takes RN_bf16(x) of row c, column c + 8 the
    // remainder x - RN_bf16(x) (at most 3 significant bits, exact in bf16), so
    // every product is exact and the two columns' sums add up to the row's
    static_assert(DT == DT_BF16 || DT == DT_F16, "16-bit activations");
    constexpr bool kSplit = DT == DT_F16;
    constexpr int kCodes = mf_chunk_codes<FMT>();        // codes per chunk
    constexpr int kSegs = kCodes / 128;                  // 128-code segments per chunk
    constexpr int kBlk = FMT == FMT_NVFP4 ? 16 : 32;     // codes per scale
    constexpr int kScB = kCodes / kBlk;                  // scale bytes per row and chunk
    constexpr int RT = mf_tiles<FMT, kWhole, NORM>();    // 16-row tiles per block
    constexpr int kRows = 16 * RT;                       // weight rows per block
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nw = (int)(blockDim.x >> 6);
    const int r16 = lane & 15;
    const int q = lane >> 4;
    const int B = (int)p.B;
    const int64_t K = p.K, N = p.N;
    const int64_t row0 = (int64_t)blockIdx.x * kRows;
    const int64_t nchunks = (K + kCodes - 1) / kCodes;
    uint8_t* wl = smem + (size_t)wave * kRows * kMfChunkBytes;
    const S* x = static_cast<const S*>(p.x);
    const uint8_t* scb = static_cast<const uint8_t*>(p.scales);

    // rows this lane loads (coalesced) and reads (operand layout), clamped
    int64_t lrow[2 * RT];
#pragma unroll
    for (int i = 0; i < 2 * RT; ++i) {
        const int64_t r = row0 + 8 * i + (lane >> 3);
        lrow[i] = r < N ? r : N - 1;
    }
    int64_t orow[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int64_t r = row0 + 16 * t + r16;
        orow[t] = r < N ? r : N - 1;
    }
    // x through a buffer resource over its B rows: a load at an offset past
    // the buffer returns zeros and makes no memory request, so the columns
    // past B (never stored) and pieces past K cost nothing and read as zeros
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<S*>(x), 0, (int)(B * K * (int64_t)sizeof(S)), kBufferWord3);
    const int xr16 = kSplit ? (r16 & 7) : r16;          // the x row of this lane's column
    const bool has = xr16 < B;
    const int xoff = (int)(xr16 * K * (int64_t)sizeof(S));
    // gamma [K] through its own resource (NORM)
    const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(NORM ? na.gamma : static_cast<const void*>(x)), 0,
        (int)(K * (int64_t)sizeof(S)), kBufferWord3);
    float ss = 0.0f;   // NORM: this lane's sum of x^2 (column r16)

    mf_f32x4_t acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] = mf_f32x4_t{0.f, 0.f, 0.f, 0.f};

    // kWhole: the block's scale rows (one contiguous range of kRows x
    // sc_per_row bytes) are staged once in LDS after the weight area, each row
    // padded by 16 bytes so the operand rows' reads hit distinct banks. The
    // 16-byte pieces are loaded here, ahead of every weight load; their LDS
    // writes wait for them alone (the counters retire in order) and happen
    // after the first chunk's loads have gone out, before one barrier.
    constexpr int kScPieces = mf_scale_pieces<FMT, kWhole, NORM>();
    const int sc_row = (int)p.sc_per_row;
    const int sc_stride = sc_row + 16;
    uint8_t* sst = smem + (size_t)nw * kRows * kMfChunkBytes;
    v4u scp[kScPieces];
    if constexpr (kWhole) {
        const int64_t base = row0 * p.sc_per_row;
        const int64_t last = N * p.sc_per_row - 16;
        const int n16 = kRows * sc_row / 16;
#pragma unroll
        for (int j = 0; j < kScPieces; ++j) {
            const int pc = tid + j * (int)blockDim.x;
            if (j == 0 || pc < n16) {
                int64_t o = base + 16 * (int64_t)(pc < n16 ? pc : n16 - 1);
                o = o < last ? o : last;   // rows past N: their results are not stored
                scp[j] = *reinterpret_cast<const v4u*>(scb + o);
            }
        }
    }
    // (1)-(2): the loads of chunk c. The first chunk's go out before the
    // scale staging's barrier, every later chunk's at the top of its turn.
    v4u raw[2 * RT];
    v4u xb[kSegs][4];
    v4u gb[NORM ? kSegs : 1][4];
    auto issue = [&](int64_t c) __attribute__((always_inline)) {
        const int64_t code0 = c * kCodes;                // first code of the chunk
        const int64_t byte0 = FMT == FMT_MXFP8 ? code0 : code0 / 2;
        // (1) weights: instruction i covers rows 8 i .. 8 i + 7 of the block;
        // lane l takes piece (l % 8) ^ g(row) of its row's 128 bytes, so row r
        // piece p lands in slot 8 (r % 8) + (p ^ g(r)), g(r) = (r / 2) % 8.
        // Pieces past the row end read its last piece (zeroed below).
#pragma unroll
        for (int i = 0; i < 2 * RT; ++i) {
            const int r = 8 * i + (lane >> 3);
            const int piece = (lane & 7) ^ ((r >> 1) & 7);
            int64_t off = byte0 + 16 * piece;
            off = off + 16 <= p.row_bytes ? off : p.row_bytes - 16;
            raw[i] = load_vec<true, v4u>(p.w + lrow[i] * p.row_bytes + off);
        }
        // (2) x: the B operand of MFMA t of segment s in lane (column r16, q)
        // holds x[r16][code0 + 128 s + 32 q + 8 t .. + 8]
        // (pieces past K enter as zeros, with their zeroed weights). Issued
        // right behind the weights, so on the first chunk they are in flight
        // across the scale staging's barrier too (issued after it, they added
        // their L2 round trip to every wave's first chunk: MXFP4 K=4096
        // N=14336 B=4 9.63 -> 8.80 us, B=8 10.10 -> 9.30 us)
#pragma unroll
        for (int s = 0; s < kSegs; ++s) {
            const int64_t k = code0 + 128 * s + 32 * q;
            const bool ok = has && (kWhole || k < K);
            const int off = ok ? xoff + (int)(k * (int64_t)sizeof(S)) : kBufferOutOfRange;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                xb[s][t] = __builtin_bit_cast(
                    v4u, __builtin_amdgcn_raw_buffer_load_b128(xrs, off + 16 * t, 0, 0));
            if constexpr (NORM) {
                const int goff = ok ? (int)(k * (int64_t)sizeof(S)) : kBufferOutOfRange;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    gb[s][t] = __builtin_bit_cast(
                        v4u, __builtin_amdgcn_raw_buffer_load_b128(grs, goff + 16 * t, 0, 0));
            }
        }
    };
    issue(wave);
    if constexpr (kWhole) {
        const int n16 = kRows * sc_row / 16;
#pragma unroll
        for (int j = 0; j < kScPieces; ++j) {
            const int pc = tid + j * (int)blockDim.x;
            if (pc < n16) {
                const int r = pc * 16 / sc_row, col = pc * 16 - r * sc_row;
                *reinterpret_cast<v4u*>(sst + r * sc_stride + col) = scp[j];
            }
        }
        __syncthreads();
    }

    for (int64_t c = wave; c < nchunks; c += nw) {
        if (c != wave) issue(c);
        const int64_t code0 = c * kCodes;                // first code of the chunk
        // (3) scales: the row's kScB bytes of this chunk
        uint32_t sw[RT][kScB / 4 > 0 ? kScB / 4 : 1];
        const int64_t e0 = code0 / kBlk;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const uint8_t* srow = scb + orow[t] * p.sc_per_row;
            if constexpr (kWhole) {
                const uint8_t* lrw = sst + (16 * t + r16) * sc_stride + e0;
                if constexpr (kScB == 16) {
                    const v4u v = *reinterpret_cast<const v4u*>(lrw);
                    sw[t][0] = v.x; sw[t][1] = v.y; sw[t][2] = v.z; sw[t][3] = v.w;
                } else if constexpr (kScB == 8) {
                    const v2u v = *reinterpret_cast<const v2u*>(lrw);
                    sw[t][0] = v.x; sw[t][1] = v.y;
                } else {
                    sw[t][0] = *reinterpret_cast<const uint32_t*>(lrw);
                }
                (void)srow;
            } else {
#pragma unroll
                for (int j = 0; j < kScB / 4; ++j) {
                    uint32_t v = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int64_t e = e0 + 4 * j + b;
                        v |= (uint32_t)srow[e < p.sc_per_row ? e : p.sc_per_row - 1] << (8 * b);
                    }
                    sw[t][j] = v;
                }
            }
        }
        // (4) stage the chunk in the wave's LDS area (in program order with
        // this wave's operand reads of the previous chunk)
#pragma unroll
        for (int i = 0; i < 2 * RT; ++i) *reinterpret_cast<v4u*>(wl + 1024 * i + 16 * lane) = raw[i];
        if constexpr (NORM) {
            // the x pieces become RN_T(x * gamma); their squares go into ss
#pragma unroll
            for (int s = 0; s < kSegs; ++s)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t xv[4] = {xb[s][t].x, xb[s][t].y, xb[s][t].z, xb[s][t].w};
                    const uint32_t gv[4] = {gb[s][t].x, gb[s][t].y, gb[s][t].z, gb[s][t].w};
                    uint32_t o[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float x0 = Store<DT>::bits_to_f32(xv[j] & 0xFFFFu);
                        const float x1 = Store<DT>::bits_to_f32(xv[j] >> 16);
                        ss = fmaf(x0, x0, ss);
                        ss = fmaf(x1, x1, ss);
                        const f32x2 pr = {x0 * Store<DT>::bits_to_f32(gv[j] & 0xFFFFu),
                                          x1 * Store<DT>::bits_to_f32(gv[j] >> 16)};
                        if constexpr (DT == DT_F16)
                            o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, f16x2_t));
                        else
                            o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2_t));
                    }
                    xb[s][t] = v4u{o[0], o[1], o[2], o[3]};
                }
        }
        if constexpr (kSplit) {
            // the f16 pieces become their bf16 head (columns 0..7) or the exact
            // remainder (columns 8..15)
            const bool tail = r16 >= 8;
#pragma unroll
            for (int s = 0; s < kSegs; ++s)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t xv[4] = {xb[s][t].x, xb[s][t].y, xb[s][t].z, xb[s][t].w};
                    uint32_t o[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const f32x2 v = {Store<DT>::bits_to_f32(xv[j] & 0xFFFFu),
                                         Store<DT>::bits_to_f32(xv[j] >> 16)};
                        const bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
                        const f32x2 r = v - __builtin_convertvector(h, f32x2);
                        const bf16x2_t l = __builtin_convertvector(r, bf16x2_t);
                        o[j] = tail ? __builtin_bit_cast(uint32_t, l) : __builtin_bit_cast(uint32_t, h);
                    }
                    xb[s][t] = v4u{o[0], o[1], o[2], o[3]};
                }
        }
        // (5) the MFMAs
#pragma unroll
        for (int s = 0; s < kSegs; ++s) {
            const bool kv = kWhole || code0 + 128 * s + 32 * q < K;
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const int r = 16 * t + r16;
                const int g = (r >> 1) & 7;
                const uint8_t* rp = wl + 1024 * (r >> 3) + 128 * (r & 7);
                // decode four codes pairs at a time into the A operand of MFMA u
                // and issue it right away, so one operand is live at a time
                auto mfma = [&](int u, uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3)
                                __attribute__((always_inline)) {
                    if constexpr (!kWhole) {
                        a0 = kv ? a0 : 0u;
                        a1 = kv ? a1 : 0u;
                        a2 = kv ? a2 : 0u;
                        a3 = kv ? a3 : 0u;
                    }
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(V8, v4u{a0, a1, a2, a3}),
                        __builtin_bit_cast(V8, xb[s][u]), acc[t], 0, 0, 0);
                };
                if constexpr (FMT == FMT_MXFP8) {
                    // the lane's 32 codes are pieces 2 q, 2 q + 1 of the row
                    const v4u lo = *reinterpret_cast<const v4u*>(rp + 16 * ((2 * q) ^ g));
                    const v4u hi = *reinterpret_cast<const v4u*>(rp + 16 * ((2 * q + 1) ^ g));
                    const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                    const float sc = __uint_as_float(((sw[t][0] >> (8 * q)) & 0xFFu) << 23);
                    static_for<0, 4>([&](auto u_c) {
                        constexpr int u = decltype(u_c)::value;
                        mfma(u,
                             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[2 * u], sc, false)),
                             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[2 * u], sc, true)),
                             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[2 * u + 1], sc, false)),
                             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[2 * u + 1], sc, true)));
                    });
                } else {
                    const v4u dv = *reinterpret_cast<const v4u*>(rp + 16 * ((4 * s + q) ^ g));
                    const uint32_t d[4] = {dv.x, dv.y, dv.z, dv.w};
                    if constexpr (FMT == FMT_MXFP4) {
                        const float sc = __uint_as_float(((sw[t][s] >> (8 * q)) & 0xFFu) << 23);
                        static_for<0, 4>([&](auto u_c) {
                            constexpr int u = decltype(u_c)::value;
                            mfma(u,
                                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[u], sc, 0)),
                                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[u], sc, 1)),
                                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[u], sc, 2)),
                                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[u], sc, 3)));
                        });
                    } else {
                        // E2M1 times its E4M3 block scale, exact in fp32 and
                        // in bf16 (at most 6 significant bits); codes 16 q ..
                        // of the segment use scale byte 2 q, the next 16 2 q + 1
                        const uint32_t sbytes = (sw[t][2 * s + (q >> 1)] >> (16 * (q & 1))) & 0xFFFFu;
                        const f32x2 scv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sbytes, 1.0f, false);
                        static_for<0, 4>([&](auto u_c) {
                            constexpr int u = decltype(u_c)::value;
                            const float scs = u < 2 ? scv.x : scv.y;
                            uint32_t o[4];
                            static_for<0, 4>([&](auto e_c) {
                                constexpr int e = decltype(e_c)::value;
                                const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[u], 1.0f, e);
                                const f32x2 pr = {v.x * scs, v.y * scs};
                                o[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2_t));
                            });
                            mfma(u, o[0], o[1], o[2], o[3]);
                        });
                    }
                }
            }
        }
    }

    // the waves' partial tiles meet in LDS (the weight areas, once every wave
    // is done with them): element (row m, column b) of wave w at
    // red[(w * 16 RT + m) * 8 + b]; lane (r16, q) holds rows 4 q .. 4 q + 3 of each tile
    float* red = reinterpret_cast<float*>(smem);
    __syncthreads();
    // NORM: lane (q, r16)'s sum of squares at ssl[(w * 4 + q) * 16 + r16],
    // after the partial tiles (inside the weight areas: 24 kRows floats per
    // wave are free there)
    float* ssl = red + nw * kRows * 8;
    if constexpr (kSplit) {
        // column c's sum plus its remainder column's (lane r16 + 8)
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t][e] = acc[t][e] + __shfl_xor(acc[t][e], 8);
    }
    if (has && (!kSplit || r16 < 8)) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[(wave * kRows + 16 * t + 4 * q + e) * 8 + r16] = acc[t][e];
        if constexpr (NORM) ssl[(wave * 4 + q) * 16 + r16] = ss;
    }
    __syncthreads();
    const float gmul = (FMT == FMT_NVFP4 && p.gscale) ? *p.gscale : 1.0f;
    for (int idx = tid; idx < kRows * B; idx += (int)blockDim.x) {
        const int m = idx / B, b = idx - (idx / B) * B;
        if (row0 + m >= N) continue;
        float v = red[m * 8 + b];
        for (int w = 1; w < nw; ++w) v += red[(w * kRows + m) * 8 + b];
        if constexpr (NORM) {
            float t2 = 0.0f;
            for (int w = 0; w < nw; ++w)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) t2 += ssl[(w * 4 + qq) * 16 + b];
            v = v * (1.0f / sqrtf(t2 / (float)K + na.eps));
        }
        if constexpr (FMT == FMT_NVFP4) v = v * gmul;
        static_cast<S*>(p.y)[(int64_t)b * N + row0 + m] = Store<DT>::from_f32(v);
    }
}

template <int DT, int FMT, bool kWhole>
__global__ __launch_bounds__((64 * mf_max_waves<FMT, kWhole>())) void qmv_mfma_kernel(LaunchParams p) {
    mfma_tile<DT, FMT, kWhole, false>(p, NormArgs{});
}

template <int DT, int FMT, bool kWhole>
__global__ __launch_bounds__((64 * mf_max_waves<FMT, kWhole>())) void qmv_mfma_norm_kernel(
    LaunchParams p, NormArgs na) {
    mfma_tile<DT, FMT, kWhole, true>(p, na);
}

// The matrix-core QMV takes bf16 activations from the batch size where it
// beats the VALU tile, measured at K=4096, N=14336 (VALU tile -> matrix
// cores, one process):
//   MXFP4  B=2 9.21 -> 8.60, B=3 10.8 -> 8.76, B=4 12.5 -> 8.86, B=8 27.7 -> 9.30 us
//   NVFP4  B=2 9.10 -> 10.81, B=3 11.07 -> 10.91, B=4 12.6 -> 10.91, B=8 28.6 -> 11.76 us
//   MXFP8  B=2 12.46 -> 15.45, B=3 13.86 -> 15.62, B=4 15.6 -> 15.76, B=8 46.2 -> 16.4 us
// (MXFP8's 128-code chunks give each wave two chunks in turn at K=4096).
// Where the one-row kernel takes a batch (K = 2048 or 4096, up to
// row_max_batch rows) it runs first; these thresholds decide the other K.
template <int FMT> constexpr int mf_min_batch() {
    return FMT == FMT_MXFP4 ? 3 : 4;
}
// f16 batches on the matrix cores, each activation row split into a bf16
// head and its exact remainder (two MFMA columns per row), from the batch size
// where that beats the VALU tile, measured at K=4096, N=14336 (VALU tile /
// matrix cores, us, one process):
//   MXFP4  B=5 14.07 / 11.22, B=6 15.89 / 11.39, B=8 25.63 / 11.74
//   NVFP4  B=5 14.25 / 16.97, B=6 16.18 / 17.13, B=8 26.73 / 17.66
//   MXFP8  B=5 17.17 / 18.28, B=6 18.41 / 18.44, B=8 42.16 / 18.72
// and B=7 17.54 (NVFP4) / 18.67 us (MXFP8) on the matrix cores
// (below B=5 the one-row kernel takes f16 batches at K = 2048 / 4096, and was
// faster there than the split operand: MXFP4 B=3 8.57 / 10.97, B=4 10.02 / 11.17).
template <int FMT> constexpr int mf_min_batch_f16() { return FMT == FMT_MXFP4 ? 5 : 7; }
template <int FMT>
inline bool use_mfma_qmv_f16(const LaunchParams& p) {
    return p.B >= mf_min_batch_f16<FMT>() && p.B <= 8 && p.K > 0 &&
           p.B * p.K * 2 < (int64_t)kBufferOutOfRange;
}
// The fused RMSNorm's f16 batches on the matrix cores: the staged
// RN_f16(x * gamma) is split as x is. From B=5 (MXFP4, NVFP4) or 6 (MXFP8),
// measured at K=4096, N=14336 (fused VALU tile / matrix cores, us):
//   MXFP4  B=5 19.04 / 13.18, B=8 31.44 / 13.97
//   NVFP4  B=5 22.52 / 17.79, B=8 32.59 / 18.08
//   MXFP8  B=5 22.34 / 22.65, B=6 24.97 / 22.86, B=8 51.73 / 23.27
template <int FMT> constexpr int mf_min_batch_norm_f16() { return FMT == FMT_MXFP8 ? 6 : 5; }
template <int FMT>
inline bool use_mfma_norm_f16(const LaunchParams& p) {
    return p.B >= mf_min_batch_norm_f16<FMT>() && p.B <= 8 && p.K > 0 &&
           p.B * p.K * 2 < (int64_t)kBufferOutOfRange;
}
template <int FMT>
inline bool use_mfma_qmv(const LaunchParams& p) {
    // (x must fit a buffer resource below kBufferOutOfRange bytes)
    return p.B >= mf_min_batch<FMT>() && p.B <= 8 && p.K > 0 &&
           p.B * p.K * 2 < (int64_t)kBufferOutOfRange;
}

template <int DT, int FMT, bool NORM>
int launch_qmv_mfma(const LaunchParams& p, const NormArgs& na, hipStream_t st) {
    constexpr int kScB = mf_chunk_codes<FMT>() / (FMT == FMT_NVFP4 ? 16 : 32);
    // whole chunks, and scale rows the block can stage in 16-byte pieces
    bool whole = p.K % mf_chunk_codes<FMT>() == 0 && p.sc_per_row % 16 == 0 &&
                       p.sc_per_row <= kMfMaxScaleRow &&
                       (reinterpret_cast<uintptr_t>(p.scales) % 16) == 0;
    (void)kScB;
    int nw = mfma_waves(p, whole ? mf_max_waves<FMT, true>() : mf_max_waves<FMT, false>());
    int rows = 16 * (whole ? mf_tiles<FMT, true, NORM>() : mf_tiles<FMT, false, NORM>());
    if (whole && (int64_t)rows * p.sc_per_row / 16 >
                     (int64_t)mf_scale_pieces<FMT, true, NORM>() * 64 * nw) {
        // the scale rows need more pieces per thread than the instance holds
        whole = false;
        nw = mfma_waves(p, mf_max_waves<FMT, false>());
        rows = 16 * mf_tiles<FMT, false, NORM>();
    }
    // W waves stage rows x 128 bytes each (the reduction reuses that area: W x
    // rows x 8 columns x 4 bytes); whole instances add the staged scale rows
    const size_t lds = (size_t)nw * rows * kMfChunkBytes +
                       (whole ? (size_t)rows * (size_t)(p.sc_per_row + 16) : 0);
    static LdsGrant granted_w, granted_p;
    const dim3 grid((unsigned)((p.N + rows - 1) / rows));
    if constexpr (NORM) {
        auto* kern = whole ? &qmv_mfma_norm_kernel<DT, FMT, true>
                           : &qmv_mfma_norm_kernel<DT, FMT, false>;
        if (const int e = allow_lds(kern, lds, whole ? granted_w : granted_p)) return e;
        hipLaunchKernelGGL(kern, grid, dim3(64 * nw), lds, st, p, na);
    } else {
        (void)na;
        auto* kern = whole ? &qmv_mfma_kernel<DT, FMT, true> : &qmv_mfma_kernel<DT, FMT, false>;
        if (const int e = allow_lds(kern, lds, whole ? granted_w : granted_p)) return e;
        hipLaunchKernelGGL(kern, grid, dim3(64 * nw), lds, st, p);
    }
    return (int)hipGetLastError();
}

template <int DT, int FMT, int BITS, int NU, int NB>
int launch_row(const LaunchParams& p, hipStream_t st) {
    constexpr int R = 2;
    const dim3 grid((unsigned)((p.N + R * kWaves - 1) / (R * kWaves)));
    hipLaunchKernelGGL((qmv_row_kernel<DT, FMT, BITS, NU, NB, R>), grid, dim3(kThreads), 0, st, p);
    return (int)hipGetLastError();
}
template <int DT, int FMT, int BITS, int NU>
int launch_row_nu(const LaunchParams& p, hipStream_t st) {
    constexpr int kMax = row_max_batch<DT, FMT>();
    switch ((int)p.B) {
        case 2: if constexpr (kMax >= 2) return launch_row<DT, FMT, BITS, NU, 2>(p, st); break;
        case 3: if constexpr (kMax >= 3) return launch_row<DT, FMT, BITS, NU, 3>(p, st); break;
        case 4: if constexpr (kMax >= 4) return launch_row<DT, FMT, BITS, NU, 4>(p, st); break;
        default: break;
    }
    return launch_row<DT, FMT, BITS, NU, 1>(p, st);
}

template <int DT, int FMT, int BITS>
int launch_qmv_t(const LaunchParams& p, hipStream_t st) {
    if constexpr (row_kernel_ok<DT, FMT, BITS>()) {
        if (p.B <= row_max_batch<DT, FMT>() && p.N > 0 && p.K > 0 && p.K % 2048 == 0 &&
            p.K / 2048 <= row_units_max<FMT>()) {
            if (p.K == 2048) return launch_row_nu<DT, FMT, BITS, 1>(p, st);
            return launch_row_nu<DT, FMT, BITS, 2>(p, st);
        }
    }
    if constexpr (DT == DT_BF16 &&
                  (FMT == FMT_MXFP4 || FMT == FMT_NVFP4 || FMT == FMT_MXFP8)) {
        if (use_mfma_qmv<FMT>(p)) return launch_qmv_mfma<DT, FMT, false>(p, NormArgs{}, st);
    }
    if constexpr (DT == DT_F16 &&
                  (FMT == FMT_MXFP4 || FMT == FMT_NVFP4 || FMT == FMT_MXFP8)) {
        if (use_mfma_qmv_f16<FMT>(p)) return launch_qmv_mfma<DT, FMT, false>(p, NormArgs{}, st);
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
// (at most min(n_experts, n_slots) of them), so each block runs a group of
// several tiles: about one round of resident blocks for the plain gather
// (64 experts, 128 slots: down projection 57.8 -> 52.4 us, affine 70.3 ->
// 64.5 us against two rounds), two for the fused gate/up pair, whose
// affine instance measured 210 -> 219 us with one.
constexpr int64_t kGatherBlocks = 2048;
constexpr int64_t kGatherPairBlocks = 8192;

// Tiles per block of a gather launch: about `target` blocks across the
// experts that can be active.
inline int64_t gather_tiles_per_block(const LaunchParams& p, int64_t n_tiles, int64_t target) {
    const int64_t active = p.n_experts < p.n_slots ? p.n_experts : p.n_slots;
    int64_t tpb = (n_tiles * active + target - 1) / target;
    if (tpb < 1) tpb = 1;
    if (tpb > n_tiles) tpb = n_tiles > 0 ? n_tiles : 1;
    return tpb;
}

// Units per lane per row of the gather's one-row-style tile loop for this
// launch (K = 2048 * NU, NU = 1 or 2, 64 lanes per row, or K = 1536 with 16
// lanes per row; 16-bit activations; MXFP4 / NVFP4 / MXFP8 or 4-bit affine
// codes; one slab of K), or 0 for the generic loop. For the other
// instantiations gather_row_nu folds the template argument to 0, so no extra
// kernel is built for them.
template <int DT, int FMT, int BITS>
constexpr bool gather_row_ok() {
    return DT != DT_F32 && (FMT == FMT_MXFP4 || FMT == FMT_NVFP4 || FMT == FMT_MXFP8 ||
                            (FMT == FMT_AFFINE && BITS == 4));
}
template <int DT, int FMT, int BITS>
constexpr int gather_row_nu(int nu) { return gather_row_ok<DT, FMT, BITS>() ? nu : 0; }
template <int DT, int FMT, int BITS>
inline int gather_row_units(const LaunchParams& p, const Geom& g) {
    if (!gather_row_ok<DT, FMT, BITS>() || p.K <= 0 || g.ks < p.K) return 0;
    if (g.lpr == 64 && (p.K == 2048 || p.K == 4096)) return (int)(p.K / 2048);
    if (g.lpr == 16 && p.K == 1536) return 3;
    return 0;
}

template <int DT, int FMT, int BITS>
int launch_gather_t(const LaunchParams& p, hipStream_t st) {
    const NoMoeArgs none{};
    constexpr int kChunk = gather_chunk_for(DT);
    Geom g = make_geom<DT, FMT, BITS>(p, kChunk, kGatherStageBytes, kGatherRows);
    g.out_rows = g.rows_per_block;
    const int64_t n_tiles = (p.N + g.out_rows - 1) / g.out_rows;
    const int64_t tpb = gather_tiles_per_block(p, n_tiles, kGatherBlocks);
    g.tiles_per_block = (int)tpb;
    const dim3 grid((unsigned)((n_tiles + tpb - 1) / tpb), (unsigned)(p.n_experts + 1));
    const size_t lds = stage_bytes<DT, FMT, BITS>(p, g);
    const int nur = gather_row_units<DT, FMT, BITS>(p, g);
    if (nur == 1)
        hipLaunchKernelGGL((gather_kernel<DT, FMT, BITS, kGatherRows, true, kGatherPlain,
                                          gather_row_nu<DT, FMT, BITS>(1)>),
                           grid, dim3(kThreads), lds, st, p, g, none);
    else if (nur == 2)
        hipLaunchKernelGGL((gather_kernel<DT, FMT, BITS, kGatherRows, true, kGatherPlain,
                                          gather_row_nu<DT, FMT, BITS>(2)>),
                           grid, dim3(kThreads), lds, st, p, g, none);
    else if (nur == 3)
        hipLaunchKernelGGL((gather_kernel<DT, FMT, BITS, kGatherRows, true, kGatherPlain,
                                          gather_row_nu<DT, FMT, BITS>(3)>),
                           grid, dim3(kThreads), lds, st, p, g, none);
    else if (g.ks >= p.K && p.K > 0)
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
    const int64_t tpb = gather_tiles_per_block(p, n_tiles, kGatherPairBlocks);
    g.tiles_per_block = (int)tpb;
    const dim3 grid((unsigned)((n_tiles + tpb - 1) / tpb), (unsigned)(p.n_experts + 1));
    const int nur = gather_row_units<DT, FMT, BITS>(p, g);
    auto* kern = nur == 1 ? &gather_kernel<DT, FMT, BITS, kGatherRows, true, kGatherSwiglu,
                                           gather_row_nu<DT, FMT, BITS>(1)>
               : nur == 2 ? &gather_kernel<DT, FMT, BITS, kGatherRows, true, kGatherSwiglu,
                                           gather_row_nu<DT, FMT, BITS>(2)>
               : nur == 3 ? &gather_kernel<DT, FMT, BITS, kGatherRows, true, kGatherSwiglu,
                                           gather_row_nu<DT, FMT, BITS>(3)>
                          : &gather_kernel<DT, FMT, BITS, kGatherRows, true, kGatherSwiglu>;
    // the static slot lists ride on top of the dynamic x stage
    static LdsGrant granted, granted1, granted2, granted3;
    if (const int e = allow_lds(kern, lds,
                                nur == 1 ? granted1 : nur == 2 ? granted2
                                         : nur == 3 ? granted3 : granted,
                                32 * 1024))
        return e;
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
