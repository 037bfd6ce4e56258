// One slice of the kernel instantiations: the dtype QMV_DT (0 f32, 1 f16,
// 2 bf16) and the format family QMV_FAM (0 affine codes of 2, 3 and 4 bits,
// 5 affine codes of 5, 6 and 8 bits; 1 MXFP4 / NVFP4 / MXFP8; 2, 3, 4 the
// symmetric block-scaled family with E8M0, FP32 and FP16 scales, QMV and
// dequant only). The affine codes take two slices because they are the
// heaviest to compile. The build compiles this file once per (dtype,
// family) pair, in parallel.
#include "qmv_kernels.cuh"

#ifndef QMV_DT
#error "QMV_DT must be defined"
#endif
#ifndef QMV_FAM
#error "QMV_FAM must be defined"
#endif

#define QMV_CAT3(a, b, c) a##b##_##c
#define QMV_PART(name, dt, fam) QMV_CAT3(name, dt, fam)

namespace qmv {
namespace {

template <template <int, int, int> class L, class... A>
int dispatch_part(const LaunchParams& p, A... a) {
#if QMV_FAM == 0
    if (p.format != FMT_AFFINE) return (int)hipErrorInvalidValue;
    switch (p.bits) {
        case 2: return L<QMV_DT, FMT_AFFINE, 2>::run(p, a...);
        case 3: return L<QMV_DT, FMT_AFFINE, 3>::run(p, a...);
        case 4: return L<QMV_DT, FMT_AFFINE, 4>::run(p, a...);
        default: return (int)hipErrorInvalidValue;
    }
#elif QMV_FAM == 5
    if (p.format != FMT_AFFINE) return (int)hipErrorInvalidValue;
    switch (p.bits) {
        case 5: return L<QMV_DT, FMT_AFFINE, 5>::run(p, a...);
        case 6: return L<QMV_DT, FMT_AFFINE, 6>::run(p, a...);
        case 8: return L<QMV_DT, FMT_AFFINE, 8>::run(p, a...);
        default: return (int)hipErrorInvalidValue;
    }
#elif QMV_FAM == 1
    switch (p.format) {
        case FMT_MXFP4: return L<QMV_DT, FMT_MXFP4, 4>::run(p, a...);
        case FMT_NVFP4: return L<QMV_DT, FMT_NVFP4, 4>::run(p, a...);
        case FMT_MXFP8: return L<QMV_DT, FMT_MXFP8, 8>::run(p, a...);
        default: return (int)hipErrorInvalidValue;
    }
#else
    constexpr int F = FMT_SB_E8M0 + (QMV_FAM - 2);
    if (p.format != F) return (int)hipErrorInvalidValue;
    switch (p.bits) {   // the element code
#if QMV_FAM != 2
        // (E2M1 and E4M3 under E8M0 are MXFP4 and MXFP8)
        case EL_E2M1: return L<QMV_DT, F, EL_E2M1>::run(p, a...);
        case EL_E4M3: return L<QMV_DT, F, EL_E4M3>::run(p, a...);
#endif
        case EL_E5M2: return L<QMV_DT, F, EL_E5M2>::run(p, a...);
        case EL_INT + 2: return L<QMV_DT, F, EL_INT + 2>::run(p, a...);
        case EL_INT + 3: return L<QMV_DT, F, EL_INT + 3>::run(p, a...);
        case EL_INT + 4: return L<QMV_DT, F, EL_INT + 4>::run(p, a...);
        case EL_INT + 5: return L<QMV_DT, F, EL_INT + 5>::run(p, a...);
        case EL_INT + 6: return L<QMV_DT, F, EL_INT + 6>::run(p, a...);
        case EL_INT + 8: return L<QMV_DT, F, EL_INT + 8>::run(p, a...);
        default: return (int)hipErrorInvalidValue;
    }
#endif
}

template <int DT, int FMT, int BITS> struct QmvL {
    static int run(const LaunchParams& p, hipStream_t s) { return launch_qmv_t<DT, FMT, BITS>(p, s); }
};
template <int DT, int FMT, int BITS> struct QmvNormL {
    static int run(const LaunchParams& p, const NormArgs& na, hipStream_t s) {
        return launch_qmv_norm_t<DT, FMT, BITS>(p, na, s);
    }
};
template <int DT, int FMT, int BITS> struct GatherL {
    static int run(const LaunchParams& p, hipStream_t s) {
        return launch_gather_t<DT, FMT, BITS>(p, s);
    }
};
template <int DT, int FMT, int BITS> struct MoeGateUpL {
    static int run(const LaunchParams& p, const MoeArgs& m, hipStream_t s) {
        return launch_moe_gate_up_t<DT, FMT, BITS>(p, m, s);
    }
};
template <int DT, int FMT, int BITS> struct MoeDownL {
    static int run(const LaunchParams& p, const MoeArgs& m, hipStream_t s) {
        return launch_moe_down_t<DT, FMT, BITS>(p, m, s);
    }
};
template <int DT, int FMT, int BITS> struct DequantL {
    static int run(const LaunchParams& p, float* out, hipStream_t s) {
        return launch_dequant_t<DT, FMT, BITS>(p, out, s);
    }
};

}  // namespace

int QMV_PART(launch_qmv_part_, QMV_DT, QMV_FAM)(const LaunchParams& p, void* stream) {
    return dispatch_part<QmvL>(p, static_cast<hipStream_t>(stream));
}
#if QMV_FAM <= 1 || QMV_FAM == 5
int QMV_PART(launch_qmv_norm_part_, QMV_DT, QMV_FAM)(const LaunchParams& p, const NormArgs& na,
                                                      void* stream) {
    return dispatch_part<QmvNormL>(p, na, static_cast<hipStream_t>(stream));
}
int QMV_PART(launch_gather_part_, QMV_DT, QMV_FAM)(const LaunchParams& p, void* stream) {
    return dispatch_part<GatherL>(p, static_cast<hipStream_t>(stream));
}
int QMV_PART(launch_moe_gate_up_part_, QMV_DT, QMV_FAM)(const LaunchParams& p, const MoeArgs& m,
                                                        void* stream) {
    return dispatch_part<MoeGateUpL>(p, m, static_cast<hipStream_t>(stream));
}
int QMV_PART(launch_moe_down_part_, QMV_DT, QMV_FAM)(const LaunchParams& p, const MoeArgs& m,
                                                     void* stream) {
    return dispatch_part<MoeDownL>(p, m, static_cast<hipStream_t>(stream));
}
#endif
int QMV_PART(launch_dequant_part_, QMV_DT, QMV_FAM)(const LaunchParams& p, float* out,
                                                     void* stream) {
    return dispatch_part<DequantL>(p, out, static_cast<hipStream_t>(stream));
}

}  // namespace qmv
