// qmm: y[M, N] = x[M, K] . W[N, K]^T for batches past the QMV's eight rows,
// on the matrix cores ("mlx 1.0.0 - quantized_nax.h", the transposed qmm:
// activations against a packed weight matrix in the same [N, K] layout as
// the matrix-vector product; "wh-iron kernel-op coverage audit", op row
// "quantized (affine_qmv / qvm / qmm)": the M-batched prefill product).
// Compiled once per 16-bit activation type (QMM_DT: bf16 or f16).
//
// A block computes a (64 * MT) x 128 tile of y over K in slices of 64 codes
// (MT = 2 when 128-row tiles still give one per compute unit, except for
// affine codes, whose group accumulators would double the registers). Per slice it copies the x tile
// into LDS and dequantizes the W tile into LDS as the activation type, one
// 32-code unit per thread; its four waves (2 x 2) then each run MT x 2 x 4
// 32x32x16 MFMAs with fp32 accumulators. The x and W
// bytes (and scales) of the next four slices are in flight in a register
// ring while a slice is computed. When the output tiles alone are too few to
// fill the chip, the K slices are split over blocks (grid z): each split
// writes fp32 partials to a caller-owned workspace and a second kernel adds
// them in split order.
//   MXFP4 / MXFP8 / NVFP4: the stored weight is code * block scale, which is
//   exact in bf16 (a power of two times at most 4 significant bits, or E2M1
//   times E4M3: at most 6) and in f16 while it lies in f16's normal range;
//   NVFP4's fp32 tensor scale multiplies the result.
//   Affine: LDS holds the integer codes (exact) and the scale and bias are
//   applied per group outside the MFMA, in fp32:
//   sum_k x q s + x b = s * (sum_k x q) + b * (sum_k x), with sum_k x per
//   row and 32-code half-slice taken from the staged x.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qmv_common.h"
#include "qmv_device.h"

#ifndef QMM_DT
#error "QMM_DT must be defined"
#endif

namespace qmv {
namespace {

constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kLd = kBK + 8;   // LDS row stride in elements (16 bytes of padding)
constexpr int kThreads = 256;

typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

template <int DT> struct Mma;
template <> struct Mma<DT_BF16> {
    typedef __bf16 v8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
    __device__ static inline f32x16 run(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<DT_F16> {
    typedef _Float16 v8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
    __device__ static inline f32x16 run(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// Two exact fp32 values as one word of the activation type (their upper
// halves for bf16: exact values need no rounding; a round-toward-zero pack
// for f16, equally exact).
template <int DT>
__device__ inline uint32_t pack2(float a, float b) {
    if constexpr (DT == DT_BF16)
        return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// The 32 weights of one unit as the activation type, into dst[0..3] (16 bytes
// each): MX codes through the scaled converts (the E8M0 byte e enters as the
// fp32 bit pattern e << 23, which those instructions read as 2^(e - 127)),
// NVFP4 codes times their E4M3 scale in fp32, affine codes as integers.
template <int DT, int FMT, int BITS>
__device__ inline void dequant_unit(const uint32_t (&w)[Fmt<FMT, BITS>::kWords],
                                    const typename Fmt<FMT, BITS>::Raw& raw, v4u* dst) {
    uint32_t p[16];
    if constexpr (FMT == FMT_MXFP4) {
        const float s = __uint_as_float(raw.e << 23);
        static_for<0, 4>([&](auto j_c) {
            constexpr int j = decltype(j_c)::value;
            static_for<0, 4>([&](auto b_c) {
                constexpr int bt = decltype(b_c)::value;
                if constexpr (DT == DT_BF16)
                    p[4 * j + bt] = __builtin_bit_cast(
                        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], s, bt));
                else
                    p[4 * j + bt] = __builtin_bit_cast(
                        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[j], s, bt));
            });
        });
    } else if constexpr (FMT == FMT_MXFP8) {
        const float s = __uint_as_float(raw.e << 23);
        static_for<0, 8>([&](auto j_c) {
            constexpr int j = decltype(j_c)::value;
            if constexpr (DT == DT_BF16) {
                p[2 * j] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], s, false));
                p[2 * j + 1] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], s, true));
            } else {
                p[2 * j] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[j], s, false));
                p[2 * j + 1] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[j], s, true));
            }
        });
    } else if constexpr (FMT == FMT_NVFP4) {
        const f32x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.e, 1.0f, false);
        static_for<0, 4>([&](auto j_c) {
            constexpr int j = decltype(j_c)::value;
            const float s = j < 2 ? sc.x : sc.y;   // codes 0..15, 16..31
            static_for<0, 4>([&](auto b_c) {
                constexpr int bt = decltype(b_c)::value;
                const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, bt);
                p[4 * j + bt] = pack2<DT>(v.x * s, v.y * s);
            });
        });
    } else {
#pragma unroll
        for (int c = 0; c < 16; ++c)
            p[c] = pack2<DT>((float)affine_code<BITS>(w, 2 * c), (float)affine_code<BITS>(w, 2 * c + 1));
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[c] = v4u{p[4 * c], p[4 * c + 1], p[4 * c + 2], p[4 * c + 3]};
}


// MT: 32-row sub-tiles per wave, so the block tile is (64 * MT) x 128.
// GATHER: rows are routed slots (x row lhs[s], expert rhs[s]); the distinct
// experts of a tile are spread over grid z, each block running the K loop on
// its expert's matrix with the x rows of other experts' slots zero.
template <int DT, int FMT, int BITS, int MT, bool GATHER>
__global__ __launch_bounds__(kThreads) void qmm_kernel(QmmParams q, int glog2) {
    using F = Fmt<FMT, BITS>;
    using S = typename Store<DT>::S;
    using V8 = typename Mma<DT>::v8;
    constexpr int W = F::kWords;
    constexpr int kUnitBytes = 4 * W;
    constexpr bool kAffine = FMT == FMT_AFFINE;
    constexpr int kSpans = kAffine ? 2 : 1;
    constexpr int kDepth = 4;   // slices in flight per block (a register ring)
    constexpr int kBM = 64 * MT;
    constexpr int kXH = 2 * MT;  // x chunks per thread and slice

    __shared__ __align__(16) uint16_t xs[kBM * kLd];
    __shared__ __align__(16) uint16_t wsm[kBN * kLd];
    __shared__ float sx[2][kBM];   // affine: sum of x over each 32-code half of the slice

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ln = lane & 31;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = q.M, N = q.N, K = q.K;
    const int64_t m0 = (int64_t)blockIdx.y * kBM;
    const int64_t n0 = (int64_t)blockIdx.x * kBN;
    const int64_t units = K >> 5;
    const int nk = (int)((K + kBK - 1) / kBK);
    // this block's split of the K slices: [kb0, kb0 + nks), nks >= 1 (grid z
    // is the split outside gather mode; a gather never splits K)
    const int per = (nk + q.splits - 1) / q.splits;
    const int kb0 = GATHER ? 0 : (int)blockIdx.z * per;
    const int nks = (kb0 + per < nk ? kb0 + per : nk) - kb0;
    const S* x = static_cast<const S*>(q.x);
    // the matrix of the current run (gather: of expert e), its scales and biases
    const uint8_t* wcur = q.w;
    const void* sccur = q.scales;
    const void* bicur = q.biases;

    // loaders: x rows tid/8 + 32 h (h < kXH), 16-byte chunk tid%8 of the slice;
    // W row tid/2 of the tile (clamped to N - 1), unit tid%2 of the slice
    const int xr = tid >> 3, xc = tid & 7;
    const int wr = tid >> 1, wu = tid & 1;
    const int64_t wrow = n0 + wr < N ? n0 + wr : N - 1;
    // x row of each of this thread's tile rows (-1: a row of zeros)
    int64_t xrow[kXH];
#pragma unroll
    for (int h = 0; h < kXH; ++h) {
        const int64_t m = m0 + xr + 32 * h;
        xrow[h] = m < M ? m : -1;
    }
    // affine: this lane's two output columns (clamped) for the scale loads
    int64_t ncol[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t n = n0 + 64 * wn + 32 * t + ln;
        ncol[t] = n < N ? n : N - 1;
    }

    struct Slice {
        v4u x[kXH];
        uint32_t w[W];
        typename F::Raw s;
        uint32_t aff[2][kSpans][2];   // affine: raw scale, bias per column tile and span
        bool valid;
    };
    auto load_slice = [&](Slice& b, int kb) __attribute__((always_inline)) {
        const int64_t k0 = (int64_t)kb * kBK;
#pragma unroll
        for (int h = 0; h < kXH; ++h) {
            const int64_t k = k0 + xc * 8;
            if (xrow[h] >= 0 && k < K) b.x[h] = *reinterpret_cast<const v4u*>(x + xrow[h] * K + k);
            else b.x[h] = v4u{0u, 0u, 0u, 0u};
        }
        const int64_t u = (k0 >> 5) + wu;
        b.valid = u < units;
        const int64_t uc = b.valid ? u : units - 1;
        load_words<W>(wcur + wrow * q.row_bytes + uc * kUnitBytes, b.w);
        if constexpr (!kAffine) {
            b.s = F::template load_raw<DT>(sccur, bicur, wrow, q.sc_per_row, uc, glog2);
        } else {
#pragma unroll
            for (int sp = 0; sp < kSpans; ++sp) {
                // group of the span's first code; a span past K reads group 0
                // and is never applied
                const int64_t kk = k0 + 32 * sp < K ? k0 + 32 * sp : 0;
                const int64_t g = kk / q.group;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    b.aff[t][sp][0] = Store<DT>::load_bits(static_cast<const S*>(sccur) +
                                                           ncol[t] * q.sc_per_row + g);
                    b.aff[t][sp][1] = Store<DT>::load_bits(static_cast<const S*>(bicur) +
                                                           ncol[t] * q.sc_per_row + g);
                }
            }
        }
    };
    auto store_slice = [&](const Slice& b) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < kXH; ++h)
            *reinterpret_cast<v4u*>(xs + (xr + 32 * h) * kLd + xc * 8) = b.x[h];
        if constexpr (kAffine) {
            // sum of this thread's 8 x values, then over the 4 threads of a
            // 32-code half (lanes differing in bits 0..1), in a fixed order
#pragma unroll
            for (int h = 0; h < kXH; ++h) {
                const uint32_t w4[4] = {b.x[h].x, b.x[h].y, b.x[h].z, b.x[h].w};
                float t = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    t += Store<DT>::bits_to_f32(w4[j] & 0xFFFFu);
                    t += Store<DT>::bits_to_f32(w4[j] >> 16);
                }
                t += __shfl_xor(t, 1);
                t += __shfl_xor(t, 2);
                if ((xc & 3) == 0) sx[xc >> 2][xr + 32 * h] = t;
            }
        }
        uint16_t* dst = wsm + wr * kLd + wu * 32;
        if (!b.valid) {
#pragma unroll
            for (int c = 0; c < 4; ++c) reinterpret_cast<v4u*>(dst)[c] = v4u{0u, 0u, 0u, 0u};
            return;
        }
        dequant_unit<DT, FMT, BITS>(b.w, b.s, reinterpret_cast<v4u*>(dst));
    };

    // accumulators per (M sub-tile, N sub-tile); affine keeps a second set
    // for the current group
    f32x16 acc[MT][2], tmp[MT][2];
#pragma unroll
    for (int tm = 0; tm < MT; ++tm)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[tm][t][i] = tmp[tm][t][i] = 0.0f;

    const uint16_t* arow = xs + (32 * MT * wm + ln) * kLd + 8 * (lane >> 5);
    const uint16_t* brow0 = wsm + (64 * wn + ln) * kLd + 8 * (lane >> 5);
    const uint16_t* brow1 = brow0 + 32 * kLd;
    // affine: a slice's scales and biases per column tile and span, as fp32
    struct Aff {
        float s[2][kSpans], b[2][kSpans];
    };
    auto aff_of = [&](const Slice& sl) __attribute__((always_inline)) {
        Aff r{};
        if constexpr (kAffine) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int sp = 0; sp < kSpans; ++sp) {
                    r.s[t][sp] = Store<DT>::bits_to_f32(sl.aff[t][sp][0]);
                    r.b[t][sp] = Store<DT>::bits_to_f32(sl.aff[t][sp][1]);
                }
        }
        return r;
    };
    // group epilogue of affine span SP (group 32: the span's half of the
    // slice; larger groups: SP = 0 and the whole slice)
    auto epilogue = [&](const Aff& af, auto sp_c, bool whole) __attribute__((always_inline)) {
        constexpr int SP = decltype(sp_c)::value;
#pragma unroll
        for (int tm = 0; tm < MT; ++tm) {
            float sxv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int ml = 32 * MT * wm + 32 * tm + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                sxv[i] = whole ? sx[0][ml] + sx[1][ml] : sx[SP][ml];
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const float s = af.s[t][SP];
                const float bb = af.b[t][SP];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    acc[tm][t][i] = fmaf(s, tmp[tm][t][i], acc[tm][t][i]);
                    acc[tm][t][i] = fmaf(bb, sxv[i], acc[tm][t][i]);
                    tmp[tm][t][i] = 0.0f;
                }
            }
        }
    };
    // the MFMAs of one staged slice (and, for affine, its group epilogues)
    auto compute = [&](const Aff& af, int kb) __attribute__((always_inline)) {
        const int64_t k0 = (int64_t)kb * kBK;
        static_for<0, 4>([&](auto ks_c) {
            constexpr int ks = decltype(ks_c)::value;
            V8 a[MT];
#pragma unroll
            for (int tm = 0; tm < MT; ++tm)
                a[tm] = *reinterpret_cast<const V8*>(arow + 32 * tm * kLd + 16 * ks);
            const V8 b0 = *reinterpret_cast<const V8*>(brow0 + 16 * ks);
            const V8 b1 = *reinterpret_cast<const V8*>(brow1 + 16 * ks);
            if constexpr (kAffine) {
#pragma unroll
                for (int tm = 0; tm < MT; ++tm) {
                    tmp[tm][0] = Mma<DT>::run(a[tm], b0, tmp[tm][0]);
                    tmp[tm][1] = Mma<DT>::run(a[tm], b1, tmp[tm][1]);
                }
                if (q.group == 32) {
                    if constexpr ((ks & 1) == 1) {
                        if (k0 + 32 * (ks >> 1) < K)
                            epilogue(af, std::integral_constant<int, (ks >> 1)>{}, false);
                    }
                } else if constexpr (ks == 3) {
                    epilogue(af, std::integral_constant<int, 0>{}, true);
                }
            } else {
#pragma unroll
                for (int tm = 0; tm < MT; ++tm) {
                    acc[tm][0] = Mma<DT>::run(a[tm], b0, acc[tm][0]);
                    acc[tm][1] = Mma<DT>::run(a[tm], b1, acc[tm][1]);
                }
            }
        });
    };

    // the K loop over this block's slices, for the current run
    auto run_k = [&]() __attribute__((always_inline)) {
        // ring of kDepth slices: slice it + d sits in ring[d]; every load is
        // issued (clamped to the split's last slice) so the number in flight is
        // the same on every path
        Slice ring[kDepth];
        static_for<0, kDepth>([&](auto d_c) {
            constexpr int d = decltype(d_c)::value;
            load_slice(ring[d], kb0 + (d < nks ? d : nks - 1));
        });
        int it = 0;
        for (; it + kDepth <= nks; it += kDepth) {
            static_for<0, kDepth>([&](auto d_c) {
                constexpr int d = decltype(d_c)::value;
                store_slice(ring[d]);
                __syncthreads();
                const Aff af = aff_of(ring[d]);
                const int nxt = it + d + kDepth;
                load_slice(ring[d], kb0 + (nxt < nks ? nxt : nks - 1));
                compute(af, kb0 + it + d);
                __syncthreads();
            });
        }
        static_for<0, kDepth>([&](auto d_c) {
            constexpr int d = decltype(d_c)::value;
            if (it + d < nks) {
                store_slice(ring[d]);
                __syncthreads();
                compute(aff_of(ring[d]), kb0 + it + d);
                __syncthreads();
            }
        });
    };

    // gather: the tile's expert ids (ids >= n_experts, and rows past the
    // end, are kNone); block z of a tile runs the tile's z-th smallest
    // expert, the last z block also every larger one, and each stores only
    // the rows of the experts it ran (block 0 also the kNone rows, as zeros)
    constexpr uint32_t kNone = 0xFFFFFFFFu;
    __shared__ uint32_t tile_e[GATHER ? kBM : 1];
    __shared__ uint32_t next_e;
    uint32_t e_sel = kNone;
    const bool last_z = blockIdx.z + 1 == gridDim.z;
    if constexpr (!GATHER) {
        run_k();
    } else {
        for (int r = tid; r < kBM; r += kThreads) {
            const int64_t sl = m0 + r;
            uint32_t e = kNone;
            if (sl < M) {
                e = q.rhs[sl];
                if ((int64_t)e >= q.n_experts) e = kNone;
            }
            tile_e[r] = e;
        }
        // smallest expert id >= lo in the tile, or kNone
        auto tile_min = [&](uint32_t lo) __attribute__((always_inline)) {
            if (tid == 0) next_e = kNone;
            __syncthreads();
            for (int r = tid; r < kBM; r += kThreads) {
                const uint32_t e = tile_e[r];
                if (e != kNone && e >= lo) atomicMin(&next_e, e);
            }
            __syncthreads();
            const uint32_t e = next_e;
            __syncthreads();   // every thread has read next_e before it is reset
            return e;
        };
        uint32_t lo = 0;
        for (unsigned z = 0; z <= blockIdx.z; ++z) {
            e_sel = tile_min(lo);
            if (e_sel == kNone) break;
            lo = e_sel + 1;
        }
        const int64_t estride_w = N * q.row_bytes;
        const int64_t estride_s =
            N * q.sc_per_row *
            (kAffine ? (int64_t)Store<DT>::kBytes : (int64_t)F::template elem_bytes<DT>());
        uint32_t e = e_sel;
        while (e != kNone) {
#pragma unroll
            for (int h = 0; h < kXH; ++h) {
                const int r = xr + 32 * h;
                const int64_t sl = m0 + r;
                int64_t xi = -1;
                if (tile_e[r] == e) {
                    const uint32_t l = q.lhs[sl];
                    if ((int64_t)l < q.n_x_rows) xi = l;
                }
                xrow[h] = xi;
            }
            wcur = q.w + (int64_t)e * estride_w;
            sccur = static_cast<const uint8_t*>(q.scales) + (int64_t)e * estride_s;
            if constexpr (kAffine)
                bicur = static_cast<const uint8_t*>(q.biases) + (int64_t)e * estride_s;
            run_k();
            if (!last_z) break;
            e = tile_min(e + 1);
        }
    }
    // gather: does this block store local row r?
    auto mine = [&](int r) __attribute__((always_inline)) {
        if constexpr (!GATHER) {
            return true;
        } else {
            const uint32_t e = tile_e[r];
            if (e == kNone) return blockIdx.z == 0;
            if (e_sel == kNone) return false;
            return last_z ? e >= e_sel : e == e_sel;
        }
    };

    const float gs = (FMT == FMT_NVFP4 && q.gscale) ? *q.gscale : 1.0f;
#pragma unroll
    for (int tm = 0; tm < MT; ++tm) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int64_t n = n0 + 64 * wn + 32 * t + ln;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int rl = 32 * MT * wm + 32 * tm + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                const int64_t m = m0 + rl;
                if (m >= M || !mine(rl)) continue;
                if (GATHER || q.splits == 1)
                    static_cast<S*>(q.y)[m * N + n] = Store<DT>::from_f32(acc[tm][t][i] * gs);
                else
                    q.ws[((int64_t)blockIdx.z * M + m) * N + n] = acc[tm][t][i];
            }
        }
    }
}

// y = sum of the K splits' partials in split order (8 loads in flight per
// pass), times NVFP4's global scale, rounded to T once
template <int DT>
__global__ __launch_bounds__(256) void qmm_reduce_kernel(QmmParams q) {
    using S = typename Store<DT>::S;
    const int64_t MN = q.M * q.N;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= MN) return;
    float t = 0.0f;
    for (int s0 = 0; s0 < q.splits; s0 += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = s0 + j < q.splits ? s0 + j : q.splits - 1;
            v[j] = q.ws[(int64_t)s * MN + i];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) t = s0 + j < q.splits ? t + v[j] : t;
    }
    if (q.format == FMT_NVFP4 && q.gscale) t *= *q.gscale;
    static_cast<S*>(q.y)[i] = Store<DT>::from_f32(t);
}

template <int DT, int FMT, int BITS, bool GATHER>
int launch_qmm_g(const QmmParams& q, hipStream_t st) {
    const int bm = qmm_block_rows(q.M, q.N, q.format);
    const dim3 grid((unsigned)((q.N + kBN - 1) / kBN), (unsigned)((q.M + bm - 1) / bm),
                    (unsigned)(GATHER ? q.runs : q.splits));
    int glog2 = 0;
    if (FMT == FMT_AFFINE) glog2 = q.group == 128 ? 2 : (q.group == 64 ? 1 : 0);
    if constexpr (FMT != FMT_AFFINE) {
        if (bm == 128)
            hipLaunchKernelGGL((qmm_kernel<DT, FMT, BITS, 2, GATHER>), grid, dim3(kThreads), 0,
                               st, q, glog2);
        else
            hipLaunchKernelGGL((qmm_kernel<DT, FMT, BITS, 1, GATHER>), grid, dim3(kThreads), 0,
                               st, q, glog2);
    } else {
        hipLaunchKernelGGL((qmm_kernel<DT, FMT, BITS, 1, GATHER>), grid, dim3(kThreads), 0, st, q,
                           glog2);
    }
    if (q.splits > 1) {
        const int64_t n = q.M * q.N;
        hipLaunchKernelGGL((qmm_reduce_kernel<DT>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           st, q);
    }
    return (int)hipGetLastError();
}

template <int DT, int FMT, int BITS>
int launch_qmm_f(const QmmParams& q, hipStream_t st) {
    return q.rhs ? launch_qmm_g<DT, FMT, BITS, true>(q, st) : launch_qmm_g<DT, FMT, BITS, false>(q, st);
}

}  // namespace

#define QMM_CAT2(a, b) a##b
#define QMM_CAT(a, b) QMM_CAT2(a, b)

int QMM_CAT(launch_qmm_dt_, QMM_DT)(const QmmParams& q, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (q.format) {
        case FMT_AFFINE:
            switch (q.bits) {
                case 2: return launch_qmm_f<QMM_DT, FMT_AFFINE, 2>(q, st);
                case 3: return launch_qmm_f<QMM_DT, FMT_AFFINE, 3>(q, st);
                case 4: return launch_qmm_f<QMM_DT, FMT_AFFINE, 4>(q, st);
                case 5: return launch_qmm_f<QMM_DT, FMT_AFFINE, 5>(q, st);
                case 6: return launch_qmm_f<QMM_DT, FMT_AFFINE, 6>(q, st);
                case 8: return launch_qmm_f<QMM_DT, FMT_AFFINE, 8>(q, st);
            }
            return (int)hipErrorInvalidValue;
        case FMT_MXFP4: return launch_qmm_f<QMM_DT, FMT_MXFP4, 4>(q, st);
        case FMT_NVFP4: return launch_qmm_f<QMM_DT, FMT_NVFP4, 4>(q, st);
        case FMT_MXFP8: return launch_qmm_f<QMM_DT, FMT_MXFP8, 8>(q, st);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace qmv
