// Device-side building blocks of the QMV kernels for gfx950 (CDNA4):
// storage-type conversions, packed-code extraction, the format decoders and
// the per-format scale handling. Included by the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qmv_common.h"

namespace qmv {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// fp32 += a.lo*b.lo + a.hi*b.hi for two packed 16-bit pairs of type DT
// (v_dot2c_f32_bf16 / v_dot2c_f32_f16: exact products, fp32 accumulation).
template <int DT>
__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (DT == DT_BF16) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), c, false);
    } else {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                      __builtin_bit_cast(f16x2_t, b), c, false);
    }
}

// The two 16-bit values of a packed pair as fp32 (exact).
template <int DT>
__device__ inline float pair_lo(uint32_t v) {
    if constexpr (DT == DT_BF16) return __uint_as_float(v << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
template <int DT>
__device__ inline float pair_hi(uint32_t v) {
    if constexpr (DT == DT_BF16) return __uint_as_float(v & 0xFFFF0000u);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// 1.0 in both halves of a pair.
template <int DT>
__device__ constexpr uint32_t pair_ones() {
    return DT == DT_BF16 ? 0x3F803F80u : 0x3C003C00u;
}

// Compile-time loop helper.
template <int I, int N, class F>
__device__ inline void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// ---------------------------------------------------------------------------
// Storage types of x / y / affine scales and biases.
// ---------------------------------------------------------------------------
template <int DT> struct Store;

template <> struct Store<DT_F32> {
    using S = float;
    static constexpr int kBytes = 4;
    __device__ static inline float load(const S* p) { return *p; }
    __device__ static inline uint32_t load_bits(const S* p) {
        return *reinterpret_cast<const uint32_t*>(p);
    }
    __device__ static inline float bits_to_f32(uint32_t b) { return __uint_as_float(b); }
    __device__ static inline S from_f32(float v) { return v; }
};

template <> struct Store<DT_F16> {
    using S = _Float16;
    static constexpr int kBytes = 2;
    __device__ static inline float load(const S* p) { return (float)*p; }
    __device__ static inline uint32_t load_bits(const S* p) {
        return *reinterpret_cast<const uint16_t*>(p);
    }
    __device__ static inline float bits_to_f32(uint32_t b) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
    }
    // v_cvt_f16_f32 rounds to nearest-even in the default mode.
    __device__ static inline S from_f32(float v) { return (_Float16)v; }
};

template <> struct Store<DT_BF16> {
    using S = uint16_t;  // raw bfloat16 bits
    static constexpr int kBytes = 2;
    __device__ static inline float load(const S* p) {
        return __uint_as_float((uint32_t)*p << 16);
    }
    __device__ static inline uint32_t load_bits(const S* p) { return *p; }
    __device__ static inline float bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
    // fp32 -> bf16, round to nearest-even; NaN stays a quiet NaN.
    __device__ static inline S from_f32(float v) {
        uint32_t u = __float_as_uint(v);
        if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (S)((u >> 16) | 0x0040u);
        u += 0x7FFFu + ((u >> 16) & 1u);
        return (S)(u >> 16);
    }
};

// Eight consecutive stored values (16 bytes for 2-byte types, 32 for f32)
// from LDS to fp32 registers.
template <int DT>
__device__ inline void lds_load8(const typename Store<DT>::S* p, float (&v)[8]) {
    if constexpr (DT == DT_F32) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else if constexpr (DT == DT_BF16) {
        const v4u a = *reinterpret_cast<const v4u*>(p);
        const uint32_t d[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(d[i] << 16);
            v[2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
        }
    } else {
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        const h8 a = *reinterpret_cast<const h8*>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
    }
}

// ---------------------------------------------------------------------------
// Scale decoders.
// ---------------------------------------------------------------------------

// E8M0 byte e -> 2^(e-127). e = 0 is the fp32 subnormal 2^-127 (f32
// denormals are kept by these kernels); e = 255 is NaN.
__device__ inline float e8m0_to_f32(uint32_t e) {
    uint32_t b = e << 23;
    b = (e == 0u) ? 0x00400000u : b;
    b = (e == 255u) ? 0x7FC00000u : b;
    return __uint_as_float(b);
}

// ---------------------------------------------------------------------------
// Packed codes. A unit is 32 consecutive codes of one row; with b-bit codes
// it is exactly b dwords, so every unit starts on a dword boundary and code j
// of the unit sits at bit j*b of the unit's little-endian bit stream.
// ---------------------------------------------------------------------------
template <int BITS>
__device__ inline uint32_t affine_code(const uint32_t* d, int j) {
    const int bit = j * BITS;
    const int w = bit >> 5;
    const int off = bit & 31;
    const uint32_t mask = (1u << BITS) - 1u;
    if (off + BITS <= 32) return (d[w] >> off) & mask;
    // the code straddles two dwords: funnel-shift the pair
    return __builtin_amdgcn_alignbit(d[w + 1], d[w], off) & mask;
}

// One vector load of a value read once (NT: the nontemporal hint, so a
// stream of weights does not displace what the caches hold for reuse).
template <bool NT, class V>
__device__ inline V load_vec(const uint8_t* p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
    else
        return *reinterpret_cast<const V*>(p);
}

// The WORDS dwords of one unit. Units of 2, 4 and 8 dwords are 8- or 16-byte
// aligned and take vector loads; the 3-, 5- and 6-dword units of 3/5/6-bit
// codes are only 4-byte aligned and take plain loads. NT applies to units of
// at most 16 bytes, where each load instruction of a wave covers whole cache
// lines; the two 16-byte halves of an 8-dword unit share their lines, and
// with the hint the 8-bit QMV ran ~10 % slower (measured), so they load plainly.
template <int WORDS, bool NT = false>
__device__ inline void load_words(const uint8_t* p, uint32_t (&d)[WORDS]) {
    if constexpr (WORDS == 4) {
        const v4u a = load_vec<NT, v4u>(p);
        d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
    } else if constexpr (WORDS == 8) {
        const v4u a = load_vec<false, v4u>(p);
        const v4u b = load_vec<false, v4u>(p + 16);
        d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
        d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
    } else if constexpr (WORDS == 2) {
        const v2u a = load_vec<NT, v2u>(p);
        d[0] = a.x; d[1] = a.y;
    } else {
        __builtin_memcpy(d, __builtin_assume_aligned(p, 4), 4 * WORDS);
    }
}

// ---------------------------------------------------------------------------
// Formats. Each defines
//   kWords            dwords of packed codes per unit of 32
//   Raw / load_raw    the per-(row, unit) scale bytes as loaded (undecoded, so
//                     a load in flight is not waited on until its use)
//   kArrays, elem_bytes, elem_of_unit, lds_raw
//                     the scale arrays as staged in LDS for a tile
//   global_raw        the same bytes read from the global arrays at a byte
//                     offset from uniform bases
//   Scale / decode    the fp32 scale data of the unit
//   decode8<SC>(d,q)  fp32 values of codes 8*SC .. 8*SC+7 of the unit
// ---------------------------------------------------------------------------
template <int FMT, int BITS> struct Fmt;

template <int BITS> struct Fmt<FMT_AFFINE, BITS> {
    static constexpr int kWords = BITS;
    static constexpr bool kNeedsSumX = true;
    static constexpr bool kTwoScales = false;
    struct Raw { uint32_t s, b; };
    struct Scale { float s, b; };
    template <int DT>
    __device__ static inline Raw load_raw(const void* sc, const void* bi, int64_t row,
                                          int64_t sc_per_row, int64_t u, int glog2) {
        using S = typename Store<DT>::S;
        const int64_t i = row * sc_per_row + (u >> glog2);
        return Raw{Store<DT>::load_bits(static_cast<const S*>(sc) + i),
                   Store<DT>::load_bits(static_cast<const S*>(bi) + i)};
    }
    template <int DT>
    __device__ static inline Scale decode(const Raw& r) {
        return Scale{Store<DT>::bits_to_f32(r.s), Store<DT>::bits_to_f32(r.b)};
    }
    // Scale staging in LDS: two arrays (scales, biases) of T, one element per
    // group of (1 << glog2) units.
    static constexpr int kArrays = 2;
    template <int DT> __host__ __device__ static constexpr int elem_bytes() {
        return Store<DT>::kBytes;
    }
    __host__ __device__ static inline int64_t elem_of_unit(int64_t u, int glog2) { return u >> glog2; }
    // raw scale of unit ul (slab-local) from the staged copy; `row` points at
    // the row's segment of the first array, `arr` is the distance to the second
    template <int DT>
    __device__ static inline Raw lds_raw(const uint8_t* row, int arr, int ul, int glog2) {
        const int o = (ul >> glog2) * Store<DT>::kBytes;
        if constexpr (Store<DT>::kBytes == 4)
            return Raw{*reinterpret_cast<const uint32_t*>(row + o),
                       *reinterpret_cast<const uint32_t*>(row + arr + o)};
        else
            return Raw{*reinterpret_cast<const uint16_t*>(row + o),
                       *reinterpret_cast<const uint16_t*>(row + arr + o)};
    }
    // raw scale of unit u from the global arrays: `row_off` is the row's
    // byte offset from both bases (a 32-bit lane offset on a uniform base)
    template <int DT>
    __device__ static inline Raw global_raw(const uint8_t* sc, const uint8_t* bi,
                                            uint32_t row_off, int u, int glog2) {
        const uint32_t o = row_off + (uint32_t)(u >> glog2) * Store<DT>::kBytes;
        using S = typename Store<DT>::S;
        return Raw{Store<DT>::load_bits(reinterpret_cast<const S*>(sc + o)),
                   Store<DT>::load_bits(reinterpret_cast<const S*>(bi + o))};
    }
    template <int SC>
    __device__ static inline void decode8(const uint32_t (&d)[kWords], float (&q)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = (float)affine_code<BITS>(d, SC * 8 + j);
    }
    // Packed 16-bit path (4-bit codes only): pair k of sub-chunk SC holds
    // codes (8SC + k, 8SC + k + 4) as the 16-bit values 1 + q/16, built by
    // placing the nibble under the leading mantissa bits of 1.0 (exact). The
    // x pairs in LDS are ordered to match: (x[k], x[k + 4]).
    template <int SC, int DT>
    __device__ static inline void pairs(const uint32_t (&d)[kWords], uint32_t (&wp)[4]) {
        static_assert(BITS == 4, "packed affine path is for 4-bit codes");
        const uint32_t w = d[SC];
        if constexpr (DT == DT_BF16) {
            // bf16 1.0 = 0x3F80; nibble at mantissa bits 6..3
            wp[0] = ((w << 3) & 0x00780078u) | 0x3F803F80u;
            wp[1] = ((w >> 1) & 0x00780078u) | 0x3F803F80u;
            wp[2] = ((w >> 5) & 0x00780078u) | 0x3F803F80u;
            wp[3] = ((w >> 9) & 0x00780078u) | 0x3F803F80u;
        } else {
            // f16 1.0 = 0x3C00; nibble at mantissa bits 9..6
            wp[0] = ((w << 6) & 0x03C003C0u) | 0x3C003C00u;
            wp[1] = ((w << 2) & 0x03C003C0u) | 0x3C003C00u;
            wp[2] = ((w >> 2) & 0x03C003C0u) | 0x3C003C00u;
            wp[3] = ((w >> 6) & 0x03C003C0u) | 0x3C003C00u;
        }
    }
    // code value of a pair half built by `pairs` (1 + q/16 -> q, exact)
    __device__ static inline float pair_code(float v) { return (v - 1.0f) * 16.0f; }
};

// E2M1 packed pairs: pair k = codes (2k, 2k+1) of the dword, as bf16 / f16
// (every E2M1 value is exact in both).
template <int DT>
__device__ inline void e2m1_pairs(const uint32_t w, uint32_t (&wp)[4]) {
    static_for<0, 4>([&](auto k_c) {
        constexpr int k = decltype(k_c)::value;
        if constexpr (DT == DT_BF16)
            wp[k] = __builtin_bit_cast(uint32_t,
                                       __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, k));
        else
            wp[k] = __builtin_bit_cast(uint32_t,
                                       __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, k));
    });
}

// E2M1 pairs: byte k of a dword holds codes 2k (low nibble) and 2k+1.
__device__ inline void decode_e2m1_8(const uint32_t word, float (&q)[8]) {
    const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
    const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
    const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
    const f32x2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
    q[0] = a.x; q[1] = a.y; q[2] = b.x; q[3] = b.y;
    q[4] = c.x; q[5] = c.y; q[6] = e.x; q[7] = e.y;
}

template <> struct Fmt<FMT_MXFP4, 4> {
    static constexpr int kWords = 4;
    static constexpr bool kNeedsSumX = false;
    static constexpr bool kTwoScales = false;
    struct Raw { uint32_t e; };
    struct Scale { float s; };
    template <int DT>
    __device__ static inline Raw load_raw(const void* sc, const void*, int64_t row,
                                          int64_t sc_per_row, int64_t u, int) {
        return Raw{static_cast<const uint8_t*>(sc)[row * sc_per_row + u]};
    }
    template <int DT>
    __device__ static inline Scale decode(const Raw& r) { return Scale{e8m0_to_f32(r.e)}; }
    // one E8M0 byte per unit
    static constexpr int kArrays = 1;
    template <int DT> __host__ __device__ static constexpr int elem_bytes() { return 1; }
    __host__ __device__ static inline int64_t elem_of_unit(int64_t u, int) { return u; }
    template <int DT>
    __device__ static inline Raw lds_raw(const uint8_t* row, int, int ul, int) {
        return Raw{row[ul]};
    }
    template <int DT>
    __device__ static inline Raw global_raw(const uint8_t* sc, const uint8_t*, uint32_t row_off,
                                            int u, int) {
        return Raw{sc[row_off + (uint32_t)u]};
    }
    template <int SC>
    __device__ static inline void decode8(const uint32_t (&d)[kWords], float (&q)[8]) {
        decode_e2m1_8(d[SC], q);
    }
    template <int SC, int DT>
    __device__ static inline void pairs(const uint32_t (&d)[kWords], uint32_t (&wp)[4]) {
        e2m1_pairs<DT>(d[SC], wp);
    }
    __device__ static inline float pair_code(float v) { return v; }
};

template <> struct Fmt<FMT_NVFP4, 4> {
    static constexpr int kWords = 4;
    static constexpr bool kNeedsSumX = false;
    static constexpr bool kTwoScales = true;   // one scale per 16 codes
    struct Raw { uint32_t e; };      // two E4M3 bytes: blocks of codes 0..15, 16..31
    struct Scale { float lo, hi; };
    template <int DT>
    __device__ static inline Raw load_raw(const void* sc, const void*, int64_t row,
                                          int64_t sc_per_row, int64_t u, int) {
        const uint8_t* p = static_cast<const uint8_t*>(sc) + row * sc_per_row + 2 * u;
        return Raw{*reinterpret_cast<const uint16_t*>(p)};
    }
    template <int DT>
    __device__ static inline Scale decode(const Raw& r) {
        const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.e, 1.0f, false);
        return Scale{v.x, v.y};
    }
    // two E4M3 bytes per unit
    static constexpr int kArrays = 1;
    template <int DT> __host__ __device__ static constexpr int elem_bytes() { return 1; }
    __host__ __device__ static inline int64_t elem_of_unit(int64_t u, int) { return 2 * u; }
    template <int DT>
    __device__ static inline Raw lds_raw(const uint8_t* row, int, int ul, int) {
        return Raw{*reinterpret_cast<const uint16_t*>(row + 2 * ul)};
    }
    template <int DT>
    __device__ static inline Raw global_raw(const uint8_t* sc, const uint8_t*, uint32_t row_off,
                                            int u, int) {
        return Raw{*reinterpret_cast<const uint16_t*>(sc + (row_off + 2u * (uint32_t)u))};
    }
    template <int SC>
    __device__ static inline void decode8(const uint32_t (&d)[kWords], float (&q)[8]) {
        decode_e2m1_8(d[SC], q);
    }
    template <int SC, int DT>
    __device__ static inline void pairs(const uint32_t (&d)[kWords], uint32_t (&wp)[4]) {
        e2m1_pairs<DT>(d[SC], wp);
    }
    __device__ static inline float pair_code(float v) { return v; }
};

template <> struct Fmt<FMT_MXFP8, 8> {
    static constexpr int kWords = 8;
    static constexpr bool kNeedsSumX = false;
    static constexpr bool kTwoScales = false;
    struct Raw { uint32_t e; };
    struct Scale { float s; };
    template <int DT>
    __device__ static inline Raw load_raw(const void* sc, const void*, int64_t row,
                                          int64_t sc_per_row, int64_t u, int) {
        return Raw{static_cast<const uint8_t*>(sc)[row * sc_per_row + u]};
    }
    template <int DT>
    __device__ static inline Scale decode(const Raw& r) { return Scale{e8m0_to_f32(r.e)}; }
    // one E8M0 byte per unit
    static constexpr int kArrays = 1;
    template <int DT> __host__ __device__ static constexpr int elem_bytes() { return 1; }
    __host__ __device__ static inline int64_t elem_of_unit(int64_t u, int) { return u; }
    template <int DT>
    __device__ static inline Raw lds_raw(const uint8_t* row, int, int ul, int) {
        return Raw{row[ul]};
    }
    template <int DT>
    __device__ static inline Raw global_raw(const uint8_t* sc, const uint8_t*, uint32_t row_off,
                                            int u, int) {
        return Raw{sc[row_off + (uint32_t)u]};
    }
    template <int SC>
    __device__ static inline void decode8(const uint32_t (&d)[kWords], float (&q)[8]) {
        // word 2*SC holds codes 8*SC .. 8*SC+3 (one byte each), word 2*SC+1 the next 4
        const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d[2 * SC], 1.0f, false);
        const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d[2 * SC], 1.0f, true);
        const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d[2 * SC + 1], 1.0f, false);
        const f32x2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d[2 * SC + 1], 1.0f, true);
        q[0] = a.x; q[1] = a.y; q[2] = b.x; q[3] = b.y;
        q[4] = c.x; q[5] = c.y; q[6] = e.x; q[7] = e.y;
    }
    // pair k = codes (8SC + 2k, 8SC + 2k + 1): bytes 2(k&1), 2(k&1)+1 of
    // word 2SC + k/2, as bf16 / f16 (every E4M3 value is exact in both)
    template <int SC, int DT>
    __device__ static inline void pairs(const uint32_t (&d)[kWords], uint32_t (&wp)[4]) {
        static_for<0, 4>([&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            const uint32_t w = d[2 * SC + (k >> 1)];
            if constexpr (DT == DT_BF16)
                wp[k] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, (k & 1) != 0));
            else
                wp[k] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, (k & 1) != 0));
        });
    }
    __device__ static inline float pair_code(float v) { return v; }
};

// Sum of v over each group of `lpr` consecutive lanes (16, 32 or 64), left in
// the group's last lane, with DPP lane movements (VALU latency; no LDS
// crossbar). Fixed order: quad swaps, the two row mirrors, then row
// broadcasts across 16-lane rows.
__device__ inline float group_sum(float v, int lpr) {
    auto dpp = [](float x, int ctrl_id) __attribute__((always_inline)) {
        int r = 0;
        const int xi = __float_as_int(x);
        switch (ctrl_id) {
            case 0: r = __builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xF, 0xF, false); break;   // quad_perm 1,0,3,2
            case 1: r = __builtin_amdgcn_update_dpp(0, xi, 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
            case 2: r = __builtin_amdgcn_update_dpp(0, xi, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
            case 3: r = __builtin_amdgcn_update_dpp(0, xi, 0x140, 0xF, 0xF, false); break;  // row_mirror
            case 4: r = __builtin_amdgcn_update_dpp(0, xi, 0x142, 0xA, 0xF, false); break;  // row_bcast:15 -> rows 1,3
            default: r = __builtin_amdgcn_update_dpp(0, xi, 0x143, 0xC, 0xF, false); break; // row_bcast:31 -> rows 2,3
        }
        return __int_as_float(r);
    };
    v += dpp(v, 0);
    v += dpp(v, 1);
    v += dpp(v, 2);
    v += dpp(v, 3);   // every lane of a 16-lane row holds the row sum
    if (lpr > 16) v += dpp(v, 4);   // rows 1, 3: sums of rows (0,1), (2,3)
    if (lpr > 32) v += dpp(v, 5);   // row 3: sum of all four rows
    return v;
}

// Which instantiations take the packed 16-bit path: 16-bit activations with
// block-scaled formats or 4-bit affine codes. kPerm: x pairs in LDS are
// (x[k], x[k+4]) instead of (x[2k], x[2k+1]).
// ---------------------------------------------------------------------------
// Symmetric block-scaled family (the rest of the Track-1 format matrix):
// element code x block scale, no zero point. EL is the element (E2M1, E4M3,
// E5M2 or a two's-complement int of width n); FMT fixes the scale storage
// (E8M0 byte, FP32 or FP16). The block (16, 32 or 64 codes along K) is a
// run-time value carried in glog2 = log2(block / 32) in {-1, 0, 1}: every unit
// gets two scales, one per half (equal for blocks of 32 and 64), so one code
// path serves all three. Integer elements under an E8M0 scale (mxint) read as
// fixed point with one integer bit: code * 2^-(n-2).
// ---------------------------------------------------------------------------
template <int FMT, int EL> struct SbFmt {
    static constexpr int kBits = element_bits(EL);
    static constexpr bool kInt = EL > EL_E5M2;
    static constexpr int kWords = kBits;
    static constexpr bool kNeedsSumX = false;
    static constexpr bool kTwoScales = true;
    static constexpr int kEB = FMT == FMT_SB_E8M0 ? 1 : (FMT == FMT_SB_F32 ? 4 : 2);
    struct Raw { uint32_t lo, hi; };
    struct Scale { float lo, hi; };
    __host__ __device__ static inline int64_t elem_lo(int64_t u, int gl) {
        return gl < 0 ? 2 * u : u >> gl;
    }
    __host__ __device__ static inline int64_t elem_hi(int64_t u, int gl) {
        return gl < 0 ? 2 * u + 1 : u >> gl;
    }
    __device__ static inline uint32_t read_elem(const uint8_t* p) {
        if constexpr (kEB == 1) return *p;
        else if constexpr (kEB == 2) return *reinterpret_cast<const uint16_t*>(p);
        else return *reinterpret_cast<const uint32_t*>(p);
    }
    template <int DT>
    __device__ static inline Raw load_raw(const void* sc, const void*, int64_t row,
                                          int64_t sc_per_row, int64_t u, int gl) {
        const uint8_t* b = static_cast<const uint8_t*>(sc) + row * sc_per_row * kEB;
        return Raw{read_elem(b + elem_lo(u, gl) * kEB), read_elem(b + elem_hi(u, gl) * kEB)};
    }
    template <int DT>
    __device__ static inline Raw global_raw(const uint8_t* sc, const uint8_t*, uint32_t row_off,
                                            int u, int gl) {
        return Raw{read_elem(sc + (row_off + (uint32_t)elem_lo(u, gl) * kEB)),
                   read_elem(sc + (row_off + (uint32_t)elem_hi(u, gl) * kEB))};
    }
    __device__ static inline float scale_of(uint32_t r) {
        if constexpr (FMT == FMT_SB_E8M0) {
            const float s = e8m0_to_f32(r);
            if constexpr (kInt) return s * __uint_as_float((uint32_t)(127 - (kBits - 2)) << 23);
            else return s;
        } else if constexpr (FMT == FMT_SB_F32) {
            return __uint_as_float(r);
        } else {
            return (float)__builtin_bit_cast(_Float16, (uint16_t)r);
        }
    }
    template <int DT>
    __device__ static inline Scale decode(const Raw& r) {
        return Scale{scale_of(r.lo), scale_of(r.hi)};
    }
    static constexpr int kArrays = 1;
    template <int DT> __host__ __device__ static constexpr int elem_bytes() { return kEB; }
    __host__ __device__ static inline int64_t elem_of_unit(int64_t u, int gl) {
        return gl < 0 ? 2 * u : u >> gl;
    }
    template <int DT>
    __device__ static inline Raw lds_raw(const uint8_t* row, int, int ul, int gl) {
        return Raw{read_elem(row + elem_lo(ul, gl) * kEB), read_elem(row + elem_hi(ul, gl) * kEB)};
    }
    template <int SC>
    __device__ static inline void decode8(const uint32_t (&d)[kWords], float (&q)[8]) {
        if constexpr (EL == EL_E2M1) {
            decode_e2m1_8(d[SC], q);
        } else if constexpr (EL == EL_E4M3 || EL == EL_E5M2) {
            f32x2 a, b, c, e;
            if constexpr (EL == EL_E4M3) {
                a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d[2 * SC], 1.0f, false);
                b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d[2 * SC], 1.0f, true);
                c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d[2 * SC + 1], 1.0f, false);
                e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d[2 * SC + 1], 1.0f, true);
            } else {
                a = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(d[2 * SC], 1.0f, false);
                b = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(d[2 * SC], 1.0f, true);
                c = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(d[2 * SC + 1], 1.0f, false);
                e = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(d[2 * SC + 1], 1.0f, true);
            }
            q[0] = a.x; q[1] = a.y; q[2] = b.x; q[3] = b.y;
            q[4] = c.x; q[5] = c.y; q[6] = e.x; q[7] = e.y;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int32_t v = (int32_t)(affine_code<kBits>(d, SC * 8 + j) << (32 - kBits));
                q[j] = (float)(v >> (32 - kBits));
            }
        }
    }
    // packed 16-bit pairs of the float elements (every E2M1 / E4M3 / E5M2 value
    // is exact in bf16 and f16)
    template <int SC, int DT>
    __device__ static inline void pairs(const uint32_t (&d)[kWords], uint32_t (&wp)[4]) {
        if constexpr (EL == EL_E2M1) {
            e2m1_pairs<DT>(d[SC], wp);
        } else {
            static_for<0, 4>([&](auto k_c) {
                constexpr int k = decltype(k_c)::value;
                const uint32_t w = d[2 * SC + (k >> 1)];
                constexpr bool hi = (k & 1) != 0;
                if constexpr (EL == EL_E4M3) {
                    if constexpr (DT == DT_BF16)
                        wp[k] = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, hi));
                    else
                        wp[k] = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, hi));
                } else {
                    if constexpr (DT == DT_BF16)
                        wp[k] = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, hi));
                    else
                        wp[k] = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, hi));
                }
            });
        }
    }
    __device__ static inline float pair_code(float v) { return v; }
};
template <int EL> struct Fmt<FMT_SB_E8M0, EL> : SbFmt<FMT_SB_E8M0, EL> {};
template <int EL> struct Fmt<FMT_SB_F32, EL> : SbFmt<FMT_SB_F32, EL> {};
template <int EL> struct Fmt<FMT_SB_F16, EL> : SbFmt<FMT_SB_F16, EL> {};

template <int FMT, int BITS, int DT> struct Packed {
    // 16-bit activations take the packed pair path for the float elements and
    // 4-bit affine codes; f32 activations and the other integers use fp32 FMAs
    static constexpr bool kOn =
        DT != DT_F32 && (FMT == FMT_AFFINE ? BITS == 4 : (FMT <= FMT_MXFP8 || BITS <= EL_E5M2));
    static constexpr bool kPerm = kOn && FMT == FMT_AFFINE;
};

}  // namespace qmv
