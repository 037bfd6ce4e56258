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

// ---------------------------------------------------------------------------
// Storage types of x / y / affine scales and biases.
// ---------------------------------------------------------------------------
template <int DT> struct Store;

template <> struct Store<DT_F32> {
    using S = float;
    static constexpr int kBytes = 4;
    __device__ static inline float load(const S* p) { return *p; }
    __device__ static inline S from_f32(float v) { return v; }
};

template <> struct Store<DT_F16> {
    using S = _Float16;
    static constexpr int kBytes = 2;
    __device__ static inline float load(const S* p) { return (float)*p; }
    // v_cvt_f16_f32 rounds to nearest-even in the default mode.
    __device__ static inline S from_f32(float v) { return (_Float16)v; }
};

template <> struct Store<DT_BF16> {
    using S = uint16_t;  // raw bfloat16 bits
    static constexpr int kBytes = 2;
    __device__ static inline float load(const S* p) {
        return __uint_as_float((uint32_t)*p << 16);
    }
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
        const uint4 a = *reinterpret_cast<const uint4*>(p);
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

// OCP E4M3 byte -> fp32 through the gfx950 FP8 converter (scale 1.0).
__device__ inline float e4m3_to_f32(uint32_t byte) {
    const f32x2 r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(byte, 1.0f, false);
    return r.x;
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

template <int WORDS>
__device__ inline void load_words(const uint8_t* p, uint32_t (&d)[WORDS]) {
    if constexpr (WORDS == 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
    } else if constexpr (WORDS == 8) {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
        d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
        d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
    } else if constexpr (WORDS == 2) {
        const uint2 a = *reinterpret_cast<const uint2*>(p);
        d[0] = a.x; d[1] = a.y;
    } else {
        __builtin_memcpy(d, __builtin_assume_aligned(p, 4), 4 * WORDS);
    }
}

// ---------------------------------------------------------------------------
// Formats. Each defines
//   kWords            dwords of packed codes per unit of 32
//   Scale             the per-(row, unit) scale data and its loader
//   decode8<SC>(d,q)  fp32 values of codes 8*SC .. 8*SC+7 of the unit
//   kFoldEvery        sub-chunks of 8 codes per scale block (4, or 2 for NVFP4)
// ---------------------------------------------------------------------------
template <int FMT, int BITS> struct Fmt;

template <int BITS> struct Fmt<FMT_AFFINE, BITS> {
    static constexpr int kWords = BITS;
    static constexpr int kFoldEvery = 4;
    static constexpr bool kNeedsSumX = true;
    struct Scale { float s, b; };
    template <int DT>
    __device__ static inline Scale load_scale(const void* sc, const void* bi, int64_t row,
                                              int64_t sc_per_row, int64_t u, int glog2) {
        using S = typename Store<DT>::S;
        const int64_t i = row * sc_per_row + (u >> glog2);
        return Scale{Store<DT>::load(static_cast<const S*>(sc) + i),
                     Store<DT>::load(static_cast<const S*>(bi) + i)};
    }
    template <int SC>
    __device__ static inline void decode8(const uint32_t (&d)[kWords], float (&q)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = (float)affine_code<BITS>(d, SC * 8 + j);
    }
};

// E2M1 pairs: byte k of a dword holds codes 2k (low nibble) and 2k+1.
template <int SC>
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
    static constexpr int kFoldEvery = 4;
    static constexpr bool kNeedsSumX = false;
    struct Scale { float s; };
    template <int DT>
    __device__ static inline Scale load_scale(const void* sc, const void*, int64_t row,
                                              int64_t sc_per_row, int64_t u, int) {
        return Scale{e8m0_to_f32(static_cast<const uint8_t*>(sc)[row * sc_per_row + u])};
    }
    template <int SC>
    __device__ static inline void decode8(const uint32_t (&d)[kWords], float (&q)[8]) {
        decode_e2m1_8<SC>(d[SC], q);
    }
};

template <> struct Fmt<FMT_NVFP4, 4> {
    static constexpr int kWords = 4;
    static constexpr int kFoldEvery = 2;
    static constexpr bool kNeedsSumX = false;
    struct Scale { float lo, hi; };  // blocks of 16: codes 0..15 and 16..31
    template <int DT>
    __device__ static inline Scale load_scale(const void* sc, const void*, int64_t row,
                                              int64_t sc_per_row, int64_t u, int) {
        const uint8_t* p = static_cast<const uint8_t*>(sc) + row * sc_per_row + 2 * u;
        const uint32_t v = *reinterpret_cast<const uint16_t*>(p);
        const f32x2 r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 1.0f, false);
        return Scale{r.x, r.y};
    }
    template <int SC>
    __device__ static inline void decode8(const uint32_t (&d)[kWords], float (&q)[8]) {
        decode_e2m1_8<SC>(d[SC], q);
    }
};

template <> struct Fmt<FMT_MXFP8, 8> {
    static constexpr int kWords = 8;
    static constexpr int kFoldEvery = 4;
    static constexpr bool kNeedsSumX = false;
    struct Scale { float s; };
    template <int DT>
    __device__ static inline Scale load_scale(const void* sc, const void*, int64_t row,
                                              int64_t sc_per_row, int64_t u, int) {
        return Scale{e8m0_to_f32(static_cast<const uint8_t*>(sc)[row * sc_per_row + u])};
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
};

// Compile-time loop helper.
template <int I, int N, class F>
__device__ inline void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

}  // namespace qmv
