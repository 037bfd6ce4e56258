// Quantize-from-float kernels: a [N, K] matrix of T values (f32 / f16 / bf16)
// into the packed formats the QMV kernels read.
//
// Sources ("wh-iron kernel-op coverage audit", section "Quantization precision
// coverage"): Track 2 encodes affine integers with a per-group min/max giving
// scale and bias; the op-coverage rows fp_quantized and kv_cache take a
// per-block maximum as the scale and round elements to the nearest value,
// saturating; the Track-1 table gives the NVFP4 two-level layout (E4M3 per 16
// plus an fp32 tensor scale). Where the pages leave a step open, the reading
// taken is stated at each kernel; every step that decides a code is a single
// fp32 operation in the stated order (IEEE round-to-nearest-even, division
// correctly rounded), so the result is defined bit for bit.
//
// Work split: each lane takes 8 consecutive elements of a row (one 16-byte
// load for 2-byte T, two for f32); the lanes of one group or block (4, 8 or 16
// lanes for affine groups of 32/64/128, 4 for MX blocks of 32, 2 for NVFP4
// blocks of 16) are adjacent in the wave and combine their minima / maxima
// with lane shuffles. 8 codes of b bits are exactly b bytes, so every lane
// writes whole bytes of the packed row.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv_common.h"
#include "qmv_device.h"

namespace qmv {
namespace {

constexpr int kQThreads = 256;

template <int DT>
__device__ inline void load8(const typename Store<DT>::S* p, float (&v)[8]) {
    if constexpr (DT == DT_F32) {
        const v4u a = *reinterpret_cast<const v4u*>(p);
        const v4u b = *reinterpret_cast<const v4u*>(p + 4);
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
        v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
        v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
        v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
    } else {
        const v4u a = *reinterpret_cast<const v4u*>(p);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = Store<DT>::bits_to_f32(w[i] & 0xFFFFu);
            v[2 * i + 1] = Store<DT>::bits_to_f32(w[i] >> 16);
        }
    }
}

// min / max / max over the L adjacent lanes of a group (L a power of two <= 16)
template <int L> __device__ inline float group_min(float v) {
#pragma unroll
    for (int o = 1; o < L; o <<= 1) v = fminf(v, __shfl_xor(v, o));
    return v;
}
template <int L> __device__ inline float group_max(float v) {
#pragma unroll
    for (int o = 1; o < L; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// floor(log2(a)) of a positive finite fp32 value, subnormals included
__device__ inline int floor_log2(float a) {
    const uint32_t u = __float_as_uint(a);
    const int ef = (int)(u >> 23);
    if (ef > 0) return ef - 127;
    return -149 + (31 - __clz((int)u));
}

// exact 2^e for -149 <= e <= 127
__device__ inline float pow2(int e) {
    if (e >= -126) return __uint_as_float((uint32_t)(e + 127) << 23);
    return __uint_as_float(1u << (e + 149));
}

// E2M1 code nearest to t (ties to the even code, saturating at 6; sign from
// t's sign bit). Magnitudes 0 .5 1 1.5 2 3 4 6 are codes 0..7; the bounds are
// the midpoints, each closed on the side of its even neighbour.
__device__ inline uint32_t e2m1_encode(float t) {
    const float m = fabsf(t);
    uint32_t c;
    if (m <= 0.25f) c = 0;
    else if (m < 0.75f) c = 1;
    else if (m <= 1.25f) c = 2;
    else if (m < 1.75f) c = 3;
    else if (m <= 2.5f) c = 4;
    else if (m < 3.5f) c = 5;
    else if (m <= 5.0f) c = 6;
    else c = 7;
    return c | ((__float_as_uint(t) >> 28) & 8u);
}

// OCP E4M3 (fn) byte nearest to t (ties to even, saturating at 448, sign from
// t's sign bit). Below 2^-6 the step is 2^-9 (subnormals, whose codes 0..8
// run straight into the first normal); above, the value is scaled exactly to
// [8, 16] units of its binade's step and rounded; a carry to 16 lands on the
// next binade's code, as the codes are contiguous.
__device__ inline uint32_t e4m3_encode(float t) {
    const float m = fabsf(t);
    uint32_t c;
    if (m >= 448.0f) {
        c = 0x7E;
    } else if (m < 0.015625f) {
        c = (uint32_t)rintf(m * 512.0f);
    } else {
        const int e = floor_log2(m);
        const float k = rintf(m * pow2(3 - e));
        c = (uint32_t)((e + 7) << 3) + (uint32_t)k - 8u;
        if (c > 0x7E) c = 0x7E;
    }
    return c | ((__float_as_uint(t) >> 24) & 0x80u);
}

__device__ inline float e4m3_decode(uint32_t byte) {
    const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(byte, 1.0f, false);
    return v.x;
}

// ---------------------------------------------------------------------------
// Affine. Per group, in fp32: lo, hi = min, max; s32 = (hi - lo) / (2^b - 1);
// the stored scale and bias are RN_T(s32) and RN_T(lo); codes are taken
// against the stored values: q = clamp(rint((w - b) / s), 0, 2^b - 1), or 0
// when the stored scale is 0.
// ---------------------------------------------------------------------------
template <int DT, int BITS, int L>
__global__ __launch_bounds__(kQThreads) void quantize_affine_kernel(
    const typename Store<DT>::S* __restrict__ w, int64_t N, int64_t K, uint8_t* __restrict__ packed,
    typename Store<DT>::S* __restrict__ scales, typename Store<DT>::S* __restrict__ biases) {
    using S = typename Store<DT>::S;
    constexpr int kGroup = 8 * L;
    const int64_t lanes_per_row = K >> 3;
    const int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
    const bool live = i < N * lanes_per_row;
    const int64_t ic = live ? i : N * lanes_per_row - 1;   // keep the group's shuffles whole
    const int64_t row = ic / lanes_per_row;
    const int64_t k0 = (ic - row * lanes_per_row) << 3;
    float v[8];
    load8<DT>(w + row * K + k0, v);
    float lo = v[0], hi = v[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
        lo = fminf(lo, v[j]);
        hi = fmaxf(hi, v[j]);
    }
    lo = group_min<L>(lo) + 0.0f;   // zero extremes count as +0
    hi = group_max<L>(hi) + 0.0f;
    constexpr float kLevels = (float)((1 << BITS) - 1);
    const float s32 = (hi - lo) / kLevels;
    const S s_st = Store<DT>::from_f32(s32);
    const S b_st = Store<DT>::from_f32(lo);
    const float s = Store<DT>::load(&s_st);
    const float b = Store<DT>::load(&b_st);
    uint64_t bitsv = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float q = 0.0f;
        if (s > 0.0f) q = fminf(fmaxf(rintf((v[j] - b) / s), 0.0f), kLevels);
        bitsv |= (uint64_t)(uint32_t)q << (j * BITS);
    }
    if (!live) return;
    uint8_t* dst = packed + row * (K * BITS / 8) + (k0 >> 3) * BITS;
    if constexpr (BITS == 2) {
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)bitsv;
    } else if constexpr (BITS == 4) {
        *reinterpret_cast<uint32_t*>(dst) = (uint32_t)bitsv;
    } else if constexpr (BITS == 8) {
        *reinterpret_cast<uint64_t*>(dst) = bitsv;
    } else if constexpr (BITS == 6) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
            reinterpret_cast<uint16_t*>(dst)[j] = (uint16_t)(bitsv >> (16 * j));
    } else {
#pragma unroll
        for (int j = 0; j < BITS; ++j) dst[j] = (uint8_t)(bitsv >> (8 * j));
    }
    if ((threadIdx.x & (L - 1)) == 0) {
        const int64_t gi = row * (K / kGroup) + k0 / kGroup;
        scales[gi] = s_st;
        biases[gi] = b_st;
    }
}

// ---------------------------------------------------------------------------
// MX (block 32, E8M0). a = max |w| of the block; byte = 0 if a == 0, else
// clamp(floor(log2 a) - emax + 127, 0, 254) with emax 2 (E2M1) or 8 (E4M3);
// element = nearest to w / 2^(byte - 127), ties to even, saturating.
// ---------------------------------------------------------------------------
template <int DT, bool kFp8>
__global__ __launch_bounds__(kQThreads) void quantize_mx_kernel(
    const typename Store<DT>::S* __restrict__ w, int64_t N, int64_t K, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ scales) {
    constexpr int L = 4;
    const int64_t lanes_per_row = K >> 3;
    const int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
    const bool live = i < N * lanes_per_row;
    const int64_t ic = live ? i : N * lanes_per_row - 1;
    const int64_t row = ic / lanes_per_row;
    const int64_t k0 = (ic - row * lanes_per_row) << 3;
    float v[8];
    load8<DT>(w + row * K + k0, v);
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[j]));
    a = group_max<L>(a);
    int e = 0;
    if (a > 0.0f) e = min(max(floor_log2(a) - (kFp8 ? 8 : 2) + 127, 0), 254);
    // w / 2^(e - 127) as w * 2^(127 - e): the reciprocal of a power of two in
    // [2^-127, 2^127] is exact in fp32 (2^-127 as a subnormal), so the product
    // is the correctly rounded quotient, bit for bit, at a fraction of the
    // cost of an IEEE division
    const float Xinv = pow2(127 - e);
    if (!live) return;
    if constexpr (kFp8) {
        uint64_t out = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) out |= (uint64_t)e4m3_encode(v[j] * Xinv) << (8 * j);
        *reinterpret_cast<uint64_t*>(packed + row * K + k0) = out;
    } else {
        uint32_t out = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) out |= e2m1_encode(v[j] * Xinv) << (4 * j);
        *reinterpret_cast<uint32_t*>(packed + row * (K / 2) + (k0 >> 1)) = out;
    }
    if ((threadIdx.x & (L - 1)) == 0) scales[row * (K / 32) + k0 / 32] = (uint8_t)e;
}

// ---------------------------------------------------------------------------
// NVFP4. global = A / 2688 with A = max |w| of the whole matrix (448 * 6: the
// largest block scale lands on E4M3's largest value). Per block of 16:
// sb = (max |w| / 6) / global, scale byte = E4M3 nearest to sb; d = decoded
// scale * global; element = E2M1 nearest to w / d (0 when d is 0).
// The matrix maximum is gathered into the caller's global-scale word (as the
// bit pattern of a non-negative float, whose integer order is its value
// order), used by the quantize pass, then replaced by the global scale.
// ---------------------------------------------------------------------------
__global__ void zero_word_kernel(uint32_t* p) { *p = 0u; }

template <int DT>
__global__ __launch_bounds__(kQThreads) void absmax_kernel(const typename Store<DT>::S* __restrict__ w,
                                                           int64_t n8, uint32_t* __restrict__ out) {
    __shared__ float part[kQThreads / 64];
    // four 8-element loads in flight per thread before any is used (one at a
    // time left the pass waiting on each load); fmaxf ignores NaN, so the
    // maximum does not depend on the order it is taken in
    constexpr int U = 4;
    const int64_t stride = (int64_t)gridDim.x * kQThreads;
    float a = 0.0f;
    int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
    for (; i + (U - 1) * stride < n8; i += U * stride) {
        float v[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) load8<DT>(w + ((i + u * stride) << 3), v[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[u][j]));
    }
    for (; i < n8; i += stride) {
        float v[8];
        load8<DT>(w + (i << 3), v);
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[j]));
    }
    a = group_max<64>(a);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = part[0];
#pragma unroll
        for (int k = 1; k < kQThreads / 64; ++k) m = fmaxf(m, part[k]);
        atomicMax(out, __float_as_uint(m));
    }
}

constexpr float kNvGlobalDiv = 448.0f * 6.0f;

template <int DT>
__global__ __launch_bounds__(kQThreads) void quantize_nvfp4_kernel(
    const typename Store<DT>::S* __restrict__ w, int64_t N, int64_t K, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ scales, const uint32_t* __restrict__ amax_bits) {
    constexpr int L = 2;
    const int64_t lanes_per_row = K >> 3;
    const int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
    const bool live = i < N * lanes_per_row;
    const int64_t ic = live ? i : N * lanes_per_row - 1;
    const int64_t row = ic / lanes_per_row;
    const int64_t k0 = (ic - row * lanes_per_row) << 3;
    const float gs = __uint_as_float(*amax_bits) / kNvGlobalDiv;
    float v[8];
    load8<DT>(w + row * K + k0, v);
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[j]));
    a = group_max<L>(a);
    const float sb = gs > 0.0f ? (a / 6.0f) / gs : 0.0f;
    const uint32_t byte = e4m3_encode(sb);
    const float d = e4m3_decode(byte) * gs;
    if (!live) return;
    uint32_t out = 0;
    if (d != 0.0f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) out |= e2m1_encode(v[j] / d) << (4 * j);
    }
    *reinterpret_cast<uint32_t*>(packed + row * (K / 2) + (k0 >> 1)) = out;
    if ((threadIdx.x & (L - 1)) == 0) scales[row * (K / 16) + k0 / 16] = (uint8_t)byte;
}

__global__ void nv_global_kernel(uint32_t* p) {
    *reinterpret_cast<float*>(p) = __uint_as_float(*p) / kNvGlobalDiv;
}

unsigned blocks_for(int64_t lanes) { return (unsigned)((lanes + kQThreads - 1) / kQThreads); }

template <int DT, int BITS>
int launch_affine_b(const QuantParams& q, hipStream_t st) {
    using S = typename Store<DT>::S;
    const dim3 grid(blocks_for(q.N * (q.K >> 3)));
    const S* w = static_cast<const S*>(q.w);
    S* s = static_cast<S*>(q.scales);
    S* b = static_cast<S*>(q.biases);
    switch (q.group) {
        case 32: hipLaunchKernelGGL((quantize_affine_kernel<DT, BITS, 4>), grid, dim3(kQThreads), 0, st, w, q.N, q.K, q.packed, s, b); break;
        case 64: hipLaunchKernelGGL((quantize_affine_kernel<DT, BITS, 8>), grid, dim3(kQThreads), 0, st, w, q.N, q.K, q.packed, s, b); break;
        case 128: hipLaunchKernelGGL((quantize_affine_kernel<DT, BITS, 16>), grid, dim3(kQThreads), 0, st, w, q.N, q.K, q.packed, s, b); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

template <int DT>
int launch_quant_t(const QuantParams& q, hipStream_t st) {
    using S = typename Store<DT>::S;
    const S* w = static_cast<const S*>(q.w);
    const dim3 grid(blocks_for(q.N * (q.K >> 3)));
    switch (q.format) {
        case FMT_AFFINE:
            switch (q.bits) {
                case 2: return launch_affine_b<DT, 2>(q, st);
                case 3: return launch_affine_b<DT, 3>(q, st);
                case 4: return launch_affine_b<DT, 4>(q, st);
                case 5: return launch_affine_b<DT, 5>(q, st);
                case 6: return launch_affine_b<DT, 6>(q, st);
                case 8: return launch_affine_b<DT, 8>(q, st);
            }
            return (int)hipErrorInvalidValue;
        case FMT_MXFP4:
            hipLaunchKernelGGL((quantize_mx_kernel<DT, false>), grid, dim3(kQThreads), 0, st, w, q.N,
                               q.K, q.packed, static_cast<uint8_t*>(q.scales));
            return (int)hipGetLastError();
        case FMT_MXFP8:
            hipLaunchKernelGGL((quantize_mx_kernel<DT, true>), grid, dim3(kQThreads), 0, st, w, q.N,
                               q.K, q.packed, static_cast<uint8_t*>(q.scales));
            return (int)hipGetLastError();
        case FMT_NVFP4: {
            uint32_t* g = reinterpret_cast<uint32_t*>(q.global_scale);
            hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, st, g);
            const int64_t n8 = q.N * (q.K >> 3);
            // about four 8-element groups per thread: 2048 blocks cover the
            // benchmark matrix; never more blocks than groups of 256 threads
            int64_t rb = (n8 + kQThreads - 1) / kQThreads;
            if (rb > 2048) rb = 2048;
            hipLaunchKernelGGL((absmax_kernel<DT>), dim3((unsigned)rb), dim3(kQThreads), 0, st, w,
                               n8, g);
            hipLaunchKernelGGL((quantize_nvfp4_kernel<DT>), grid, dim3(kQThreads), 0, st, w, q.N, q.K,
                               q.packed, static_cast<uint8_t*>(q.scales), g);
            hipLaunchKernelGGL(nv_global_kernel, dim3(1), dim3(1), 0, st, g);
            return (int)hipGetLastError();
        }
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_quantize(const QuantParams& q, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (q.dtype) {
        case DT_F32: return launch_quant_t<DT_F32>(q, st);
        case DT_F16: return launch_quant_t<DT_F16>(q, st);
        case DT_BF16: return launch_quant_t<DT_BF16>(q, st);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace qmv
