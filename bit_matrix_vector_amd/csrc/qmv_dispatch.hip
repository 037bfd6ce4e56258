// Routes a validated launch to the translation unit that holds its kernel
// instances, and launches the device codecs.
#include "qmv_kernels.cuh"

namespace qmv {

#define QMV_DECL_SB(dt, fam)                                                            \
    int launch_qmv_part_##dt##_##fam(const LaunchParams&, void*);                       \
    int launch_dequant_part_##dt##_##fam(const LaunchParams&, float*, void*);
QMV_DECL_SB(0, 2) QMV_DECL_SB(0, 3) QMV_DECL_SB(0, 4) QMV_DECL_SB(1, 2) QMV_DECL_SB(1, 3)
QMV_DECL_SB(1, 4) QMV_DECL_SB(2, 2) QMV_DECL_SB(2, 3) QMV_DECL_SB(2, 4)
#undef QMV_DECL_SB

#define QMV_DECL_PART(dt, fam)                                                          \
    int launch_qmv_part_##dt##_##fam(const LaunchParams&, void*);                       \
    int launch_qmv_norm_part_##dt##_##fam(const LaunchParams&, const NormArgs&, void*);  \
    int launch_gather_part_##dt##_##fam(const LaunchParams&, void*);                    \
    int launch_moe_gate_up_part_##dt##_##fam(const LaunchParams&, const MoeArgs&, void*); \
    int launch_moe_down_part_##dt##_##fam(const LaunchParams&, const MoeArgs&, void*);  \
    int launch_dequant_part_##dt##_##fam(const LaunchParams&, float*, void*);
QMV_DECL_PART(0, 0) QMV_DECL_PART(0, 1) QMV_DECL_PART(1, 0)
QMV_DECL_PART(1, 1) QMV_DECL_PART(2, 0) QMV_DECL_PART(2, 1)
QMV_DECL_PART(0, 5) QMV_DECL_PART(1, 5) QMV_DECL_PART(2, 5)
#undef QMV_DECL_PART

// affine codes of 5, 6 and 8 bits live in slice 5, those of 2, 3 and 4 bits
// in slice 0, MXFP4 / NVFP4 / MXFP8 in slice 1
#define QMV_ROUTE(name, ...)                                                            \
    do {                                                                                \
        if (p.format == FMT_AFFINE && p.bits >= 5) {                                    \
            switch (p.dtype) {                                                          \
                case 0: return name##_0_5(__VA_ARGS__);                                 \
                case 1: return name##_1_5(__VA_ARGS__);                                 \
                case 2: return name##_2_5(__VA_ARGS__);                                 \
                default: return (int)hipErrorInvalidValue;                              \
            }                                                                           \
        }                                                                               \
        const int fam = p.format == FMT_AFFINE ? 0 : 1;                                 \
        switch (p.dtype * 2 + fam) {                                                    \
            case 0: return name##_0_0(__VA_ARGS__);                                     \
            case 1: return name##_0_1(__VA_ARGS__);                                     \
            case 2: return name##_1_0(__VA_ARGS__);                                     \
            case 3: return name##_1_1(__VA_ARGS__);                                     \
            case 4: return name##_2_0(__VA_ARGS__);                                     \
            case 5: return name##_2_1(__VA_ARGS__);                                     \
            default: return (int)hipErrorInvalidValue;                                  \
        }                                                                               \
    } while (0)

// The symmetric block-scaled family (QMV and dequant only): one slice per
// (dtype, scale storage).
#define QMV_ROUTE_SB(name, ...)                                                         \
    do {                                                                                \
        switch (p.dtype * 3 + (p.format - FMT_SB_E8M0)) {                               \
            case 0: return name##_0_2(__VA_ARGS__);                                     \
            case 1: return name##_0_3(__VA_ARGS__);                                     \
            case 2: return name##_0_4(__VA_ARGS__);                                     \
            case 3: return name##_1_2(__VA_ARGS__);                                     \
            case 4: return name##_1_3(__VA_ARGS__);                                     \
            case 5: return name##_1_4(__VA_ARGS__);                                     \
            case 6: return name##_2_2(__VA_ARGS__);                                     \
            case 7: return name##_2_3(__VA_ARGS__);                                     \
            case 8: return name##_2_4(__VA_ARGS__);                                     \
            default: return (int)hipErrorInvalidValue;                                  \
        }                                                                               \
    } while (0)

int launch_qmv_norm(const LaunchParams& p, const NormArgs& na, void* stream) {
    if (p.format >= FMT_SB_E8M0) return (int)hipErrorInvalidValue;
    QMV_ROUTE(launch_qmv_norm_part, p, na, stream);
}

int launch_qmv(const LaunchParams& p, void* stream) {
    if (p.format >= FMT_SB_E8M0) QMV_ROUTE_SB(launch_qmv_part, p, stream);
    QMV_ROUTE(launch_qmv_part, p, stream);
}

int launch_gather(const LaunchParams& p, void* stream) {
    if (p.format >= FMT_SB_E8M0) return (int)hipErrorInvalidValue;
    QMV_ROUTE(launch_gather_part, p, stream);
}

int launch_moe_gate_up(const LaunchParams& p, const MoeArgs& m, void* stream) {
    if (p.format >= FMT_SB_E8M0) return (int)hipErrorInvalidValue;
    QMV_ROUTE(launch_moe_gate_up_part, p, m, stream);
}

int launch_moe_down(const LaunchParams& p, const MoeArgs& m, void* stream) {
    if (p.format >= FMT_SB_E8M0) return (int)hipErrorInvalidValue;
    QMV_ROUTE(launch_moe_down_part, p, m, stream);
}

int launch_qvm_dt_0(const QvmParams&, void*);
int launch_qvm_dt_1(const QvmParams&, void*);
int launch_qvm_dt_2(const QvmParams&, void*);

int launch_qvm(const QvmParams& q, void* stream) {
    switch (q.dtype) {
        case DT_F32: return launch_qvm_dt_0(q, stream);
        case DT_F16: return launch_qvm_dt_1(q, stream);
        case DT_BF16: return launch_qvm_dt_2(q, stream);
    }
    return (int)hipErrorInvalidValue;
}

int launch_qmm_dt_1(const QmmParams&, void*);
int launch_qmm_dt_2(const QmmParams&, void*);

int launch_qmm(const QmmParams& q, void* stream) {
    switch (q.dtype) {
        case DT_F16: return launch_qmm_dt_1(q, stream);
        case DT_BF16: return launch_qmm_dt_2(q, stream);
    }
    return (int)hipErrorInvalidValue;
}

namespace {
__global__ void zero_fill_kernel(uint16_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * 256)
        p[i] = 0;
}
}  // namespace

int launch_zero_fill(void* p, int64_t bytes, void* stream) {
    const int64_t n = bytes / 2;
    if (n == 0) return 0;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint16_t*>(p), n);
    return (int)hipGetLastError();
}

int launch_dequant_device(const LaunchParams& p, float* out, void* stream) {
    if (p.format >= FMT_SB_E8M0) QMV_ROUTE_SB(launch_dequant_part, p, out, stream);
    QMV_ROUTE(launch_dequant_part, p, out, stream);
}

int launch_unpack_device(const uint8_t* packed, int64_t rows, int64_t K, int bits,
                         uint8_t* codes, void* stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t n = rows * (K >> 5);
    const dim3 grid((unsigned)((n + 255) / 256));
    switch (bits) {
#define QMV_UNPACK(b)                                                                     \
    case b:                                                                               \
        hipLaunchKernelGGL((unpack_kernel<b>), grid, dim3(256), 0, st, packed, rows, K, codes); \
        break;
        QMV_UNPACK(2) QMV_UNPACK(3) QMV_UNPACK(4) QMV_UNPACK(5) QMV_UNPACK(6) QMV_UNPACK(8)
#undef QMV_UNPACK
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

const char* hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace qmv
