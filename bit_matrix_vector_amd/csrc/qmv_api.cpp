// Host side of the C ABI declared in include/qmv.h: argument validation,
// variant selection, error reporting and the host codecs. Validation is pure
// host code and runs before any HIP call, so a rejected call touches no
// device state and no output.

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/qmv.h"
#include "qmv_common.h"

namespace {

thread_local char g_last_error[512] = "";

qmv_status_t fail(qmv_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int dtype_bytes(int dtype) { return dtype == QMV_F32 ? 4 : 2; }

bool valid_bits(int bits) {
    return bits == 2 || bits == 3 || bits == 4 || bits == 5 || bits == 6 || bits == 8;
}

qmv_status_t launch_status(int err, const char* what) {
    if (err == 0) return QMV_OK;
    return fail(QMV_ERR_HIP, "%s: HIP launch failed: %s", what, qmv::hip_error_string(err));
}

// Checks shared by every compute call. `block` is the scale block length.
qmv_status_t check_common(const char* fn, int dtype, int64_t B, int64_t K, int64_t N,
                          int64_t max_b) {
    if (dtype != QMV_F32 && dtype != QMV_F16 && dtype != QMV_BF16)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: dtype %d is not QMV_F32/F16/BF16", fn, dtype);
    if (B < 0 || K < 0 || N < 0)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: negative size (B=%lld K=%lld N=%lld)", fn,
                    (long long)B, (long long)K, (long long)N);
    if (B > max_b)
        return fail(QMV_ERR_UNSUPPORTED, "%s: B=%lld exceeds the decode batch limit %lld", fn,
                    (long long)B, (long long)max_b);
    if (K % 32)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: K=%lld is not a multiple of 32", fn,
                    (long long)K);
    // kernels address a tile's rows with 32-bit offsets from the tile's first
    // row: up to 64 rows of K bytes stay below 2^30 with K <= 2^24
    if (K > (int64_t)1 << 24 || N > (int64_t)1 << 28)
        return fail(QMV_ERR_UNSUPPORTED, "%s: K above 2^24 or N above 2^28", fn);
    return QMV_OK;
}

// Bytes of one scale element of a block-scaled format.
int scale_bytes(int format) {
    return format == QMV_NVFP4 || format == QMV_SB_F16 ? 2 : (format == QMV_SB_F32 ? 4 : 1);
}

qmv_status_t check_ptr(const char* fn, const char* name, const void* p, bool needed,
                       uintptr_t align) {
    if (!needed) return QMV_OK;
    if (p == nullptr) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: %s is NULL", fn, name);
    if (!aligned(p, align))
        return fail(QMV_ERR_MISALIGNED, "%s: %s is not %u-byte aligned", fn, name,
                    (unsigned)align);
    return QMV_OK;
}

#define QMV_TRY(expr)                         \
    do {                                      \
        qmv_status_t _st = (expr);            \
        if (_st != QMV_OK) return _st;        \
    } while (0)

// Fill the format-dependent geometry of a launch.
qmv_status_t format_geometry(const char* fn, int format, int bits, int group, int64_t K,
                             qmv::LaunchParams& lp) {
    lp.format = format;
    switch (format) {
        case QMV_AFFINE:
            if (!valid_bits(bits))
                return fail(QMV_ERR_UNSUPPORTED, "%s: bits=%d not in {2,3,4,5,6,8}", fn, bits);
            if (group != 32 && group != 64 && group != 128)
                return fail(QMV_ERR_UNSUPPORTED, "%s: group_size=%d not in {32,64,128}", fn,
                            group);
            if (K % group)
                return fail(QMV_ERR_INVALID_ARGUMENT, "%s: K=%lld not a multiple of group %d",
                            fn, (long long)K, group);
            lp.bits = bits;
            lp.group = group;
            lp.row_bytes = K * bits / 8;
            lp.sc_per_row = K / group;
            return QMV_OK;
        case QMV_MXFP4:
            lp.bits = 4; lp.group = 32; lp.row_bytes = K / 2; lp.sc_per_row = K / 32;
            return QMV_OK;
        case QMV_NVFP4:
            lp.bits = 4; lp.group = 16; lp.row_bytes = K / 2; lp.sc_per_row = K / 16;
            return QMV_OK;
        case QMV_MXFP8:
            lp.bits = 8; lp.group = 32; lp.row_bytes = K; lp.sc_per_row = K / 32;
            return QMV_OK;
        case QMV_SB_E8M0:
        case QMV_SB_F32:
        case QMV_SB_F16: {
            // `bits` is the element code, `group` the block (the format table
            // of qmv_fp_block)
            const int el = bits;
            const bool is_int = el >= QMV_EL_INT + 2 && el <= QMV_EL_INT + 8 &&
                                valid_bits(el - QMV_EL_INT);
            const bool is_fp = el == QMV_EL_E2M1 || el == QMV_EL_E4M3 || el == QMV_EL_E5M2;
            bool ok;
            if (format == QMV_SB_E8M0)
                ok = group == 32 && (is_int || el == QMV_EL_E5M2);
            else
                ok = (group == 16 && el == QMV_EL_E4M3) || (group == 32 && is_fp) ||
                     (group == 64 && is_int);
            if (!ok)
                return fail(QMV_ERR_UNSUPPORTED,
                            "%s: element %d with block %d is not a format of family %d", fn, el,
                            group, format);
            if (K % group)
                return fail(QMV_ERR_INVALID_ARGUMENT, "%s: K=%lld not a multiple of block %d",
                            fn, (long long)K, group);
            lp.bits = el;
            lp.group = group;
            lp.row_bytes = K * qmv::element_bits(el) / 8;
            lp.sc_per_row = K / group;
            return QMV_OK;
        }
        default:
            return fail(QMV_ERR_INVALID_ARGUMENT, "%s: unknown format %d", fn, format);
    }
}

qmv_status_t run_qmv(const char* fn, void* stream, int dtype, int format, int bits, int group,
                     int64_t B, int64_t K, int64_t N, const void* x, const uint8_t* w,
                     const void* scales, const void* biases, const float* gscale, void* y) {
    QMV_TRY(check_common(fn, dtype, B, K, N, 8));
    qmv::LaunchParams lp{};
    lp.dtype = dtype;
    QMV_TRY(format_geometry(fn, format, bits, group, K, lp));
    if (B == 0 || N == 0) return QMV_OK;
    const int tb = dtype_bytes(dtype);
    const bool has_k = K > 0;
    QMV_TRY(check_ptr(fn, "y", y, true, tb));
    QMV_TRY(check_ptr(fn, "x", x, has_k, 16));
    QMV_TRY(check_ptr(fn, "w", w, has_k, 16));
    if (format == QMV_AFFINE) {
        QMV_TRY(check_ptr(fn, "scales", scales, has_k, tb));
        QMV_TRY(check_ptr(fn, "biases", biases, has_k, tb));
    } else {
        QMV_TRY(check_ptr(fn, "scales", scales, has_k, scale_bytes(format)));
    }
    QMV_TRY(check_ptr(fn, "global_scale", gscale, gscale != nullptr, 4));
    if (x && y && has_k) {
        const uintptr_t xs = (uintptr_t)x, xe = xs + (uintptr_t)(B * K * tb);
        const uintptr_t ys = (uintptr_t)y, ye = ys + (uintptr_t)(B * N * tb);
        if (xs < ye && ys < xe)
            return fail(QMV_ERR_INVALID_ARGUMENT, "%s: x and y overlap", fn);
    }
    lp.B = B; lp.K = K; lp.N = N;
    lp.x = x; lp.w = w; lp.scales = scales; lp.biases = biases; lp.gscale = gscale; lp.y = y;
    return launch_status(qmv::launch_qmv(lp, stream), fn);
}

// Checks of an expert-stacked weights struct; fills the launch's format
// geometry and weight pointers.
qmv_status_t check_weights(const char* fn, const char* what, int dtype, const qmv_weights_t* wt,
                           qmv::LaunchParams& lp) {
    if (wt == nullptr)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: %s weights struct is NULL", fn, what);
    if (wt->n_experts < 0) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: negative count", fn);
    if (wt->n_experts > 65534)
        return fail(QMV_ERR_UNSUPPORTED, "%s: n_experts too large", fn);
    QMV_TRY(check_common(fn, dtype, 1, wt->K, wt->N, 1));
    lp.dtype = dtype;
    QMV_TRY(format_geometry(fn, wt->format, wt->bits, wt->group_size, wt->K, lp));
    if (wt->format >= QMV_SB_E8M0)
        return fail(QMV_ERR_UNSUPPORTED, "%s: the MoE block takes the affine, MXFP4, NVFP4 and "
                    "MXFP8 formats", fn);
    const int tb = dtype_bytes(dtype);
    const bool has_w = wt->K > 0 && wt->N > 0 && wt->n_experts > 0;
    QMV_TRY(check_ptr(fn, "w", wt->w, has_w, 16));
    if (wt->format == QMV_AFFINE) {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, has_w, tb));
        QMV_TRY(check_ptr(fn, "biases", wt->biases, has_w, tb));
    } else {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, has_w, scale_bytes(wt->format)));
    }
    QMV_TRY(check_ptr(fn, "global_scale", wt->global_scale, wt->global_scale != nullptr, 4));
    lp.K = wt->K; lp.N = wt->N; lp.n_experts = wt->n_experts;
    lp.w = wt->w; lp.scales = wt->scales; lp.biases = wt->biases;
    lp.gscale = wt->format == QMV_NVFP4 ? wt->global_scale : nullptr;
    return QMV_OK;
}

qmv_status_t run_quantize(const char* fn, void* stream, int dtype, int format, int bits,
                          int group, int64_t N, int64_t K, const void* w, uint8_t* packed,
                          void* scales, void* biases, float* gscale) {
    QMV_TRY(check_common(fn, dtype, 1, K, N, 1));
    qmv::LaunchParams lp{};
    QMV_TRY(format_geometry(fn, format, bits, group, K, lp));
    if (N == 0 || K == 0) return QMV_OK;
    const int tb = dtype_bytes(dtype);
    QMV_TRY(check_ptr(fn, "w", w, true, 16));
    QMV_TRY(check_ptr(fn, "packed", packed, true, 16));
    if (format == QMV_AFFINE) {
        QMV_TRY(check_ptr(fn, "scales", scales, true, tb));
        QMV_TRY(check_ptr(fn, "biases", biases, true, tb));
    } else {
        QMV_TRY(check_ptr(fn, "scales", scales, true, 1));
    }
    QMV_TRY(check_ptr(fn, "global_scale", gscale, format == QMV_NVFP4, 4));
    qmv::QuantParams q{};
    q.dtype = dtype; q.format = format; q.bits = lp.bits; q.group = lp.group;
    q.N = N; q.K = K; q.w = w; q.packed = packed; q.scales = scales; q.biases = biases;
    q.global_scale = gscale;
    return launch_status(qmv::launch_quantize(q, stream), fn);
}

}  // namespace

extern "C" {

qmv_status_t qmv_moe_gate_up_swiglu(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* gate,
                                    const qmv_weights_t* up, const void* x, int64_t n_tokens,
                                    const uint32_t* expert_ids, int64_t top_k, float clamp,
                                    void* mid) {
    const char* fn = "qmv_moe_gate_up_swiglu";
    qmv::LaunchParams lp{};
    QMV_TRY(check_weights(fn, "gate", dtype, gate, lp));
    qmv::LaunchParams lu{};
    QMV_TRY(check_weights(fn, "up", dtype, up, lu));
    if (gate->format != up->format || gate->N != up->N || gate->K != up->K ||
        gate->n_experts != up->n_experts ||
        (gate->format == QMV_AFFINE && (gate->bits != up->bits ||
                                        gate->group_size != up->group_size)))
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: gate and up weights differ in layout", fn);
    if (n_tokens < 0 || top_k < 1)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: n_tokens >= 0 and top_k >= 1 required", fn);
    if (n_tokens * top_k > ((int64_t)1 << 31))
        return fail(QMV_ERR_UNSUPPORTED, "%s: too many slots", fn);
    const int tb = dtype_bytes(dtype);
    if (2 * gate->K * tb > 64 * 1024)
        return fail(QMV_ERR_UNSUPPORTED, "%s: K=%lld too large (two x rows of K must fit 64 KB)",
                    fn, (long long)gate->K);
    if (n_tokens == 0 || gate->N == 0) return QMV_OK;
    QMV_TRY(check_ptr(fn, "mid", mid, true, tb));
    QMV_TRY(check_ptr(fn, "expert_ids", expert_ids, true, 4));
    QMV_TRY(check_ptr(fn, "x", x, gate->K > 0, 16));
    if (!(clamp == clamp)) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: clamp is NaN", fn);
    lp.B = 1; lp.x = x; lp.y = mid;
    lp.n_x_rows = n_tokens; lp.n_slots = n_tokens * top_k;
    lp.rhs = expert_ids; lp.lhs = nullptr;
    qmv::MoeArgs ma{};
    ma.w2 = lu.w; ma.scales2 = lu.scales; ma.biases2 = lu.biases; ma.gscale2 = lu.gscale;
    ma.top_k = top_k; ma.act_clamp = clamp;
    if (gate->K == 0)   // empty projections: silu(0) * 0 = 0 for every slot
        return launch_status(qmv::launch_zero_fill(mid, n_tokens * top_k * gate->N * tb, stream),
                             fn);
    return launch_status(qmv::launch_moe_gate_up(lp, ma, stream), fn);
}

qmv_status_t qmv_moe_down_reduce(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* down,
                                 const void* mid, int64_t n_tokens, const uint32_t* expert_ids,
                                 const float* route_weights, int64_t top_k, void* y) {
    const char* fn = "qmv_moe_down_reduce";
    qmv::LaunchParams lp{};
    QMV_TRY(check_weights(fn, "down", dtype, down, lp));
    if (n_tokens < 0 || top_k < 1)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: n_tokens >= 0 and top_k >= 1 required", fn);
    const int tb = dtype_bytes(dtype);
    if (top_k > 16 || top_k * down->K * tb > 64 * 1024)
        return fail(QMV_ERR_UNSUPPORTED,
                    "%s: top_k=%lld with K=%lld exceeds the staging limit (top_k <= 16, "
                    "top_k * K * sizeof(T) <= 64 KB)", fn, (long long)top_k, (long long)down->K);
    if (n_tokens > 65535) return fail(QMV_ERR_UNSUPPORTED, "%s: n_tokens above 65535", fn);
    if (n_tokens == 0 || down->N == 0) return QMV_OK;
    QMV_TRY(check_ptr(fn, "y", y, true, tb));
    QMV_TRY(check_ptr(fn, "expert_ids", expert_ids, true, 4));
    QMV_TRY(check_ptr(fn, "route_weights", route_weights, true, 4));
    QMV_TRY(check_ptr(fn, "mid", mid, down->K > 0, 16));
    lp.B = 1; lp.x = mid; lp.y = y;
    lp.n_x_rows = n_tokens; lp.n_slots = n_tokens * top_k;
    lp.rhs = expert_ids;
    qmv::MoeArgs ma{};
    ma.top_k = top_k; ma.route_w = route_weights;
    if (down->K == 0) {
        // empty sums: y = 0 (the plain kernel with no slots of any expert)
        lp.n_experts = 0; lp.lhs = nullptr;
    }
    return launch_status(qmv::launch_moe_down(lp, ma, stream), fn);
}

size_t qmv_qvm_workspace_bytes(int64_t B, int64_t K, int64_t N) {
    if (B <= 0 || K <= 0 || N <= 0) return 0;
    return (size_t)qmv::qvm_splits(B, K, N, nullptr) * (size_t)B * (size_t)K * sizeof(float);
}

// qvm with the caller's workspace, or (library_scratch) with the library's
// device scratch, looked up only after every argument has been validated.
static qmv_status_t qvm_impl(const char* fn, void* stream, int dtype, const qmv_weights_t* wt,
                             int64_t B, const void* x, void* y, void* workspace,
                             size_t workspace_bytes, bool library_scratch) {
    if (wt == nullptr) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: weights struct is NULL", fn);
    if (wt->n_experts != 1)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: n_experts must be 1", fn);
    QMV_TRY(check_common(fn, dtype, B, wt->K, wt->N, 8));
    qmv::LaunchParams lp{};
    QMV_TRY(format_geometry(fn, wt->format, wt->bits, wt->group_size, wt->K, lp));
    if (wt->format >= QMV_SB_E8M0)
        return fail(QMV_ERR_UNSUPPORTED, "%s: qvm takes the affine, MXFP4, NVFP4 and MXFP8 "
                    "formats", fn);
    if (B == 0 || wt->K == 0) return QMV_OK;
    const int tb = dtype_bytes(dtype);
    QMV_TRY(check_ptr(fn, "y", y, true, tb));
    if (wt->N == 0)   // empty sums
        return launch_status(qmv::launch_zero_fill(y, B * wt->K * tb, stream), fn);
    QMV_TRY(check_ptr(fn, "x", x, true, tb));
    QMV_TRY(check_ptr(fn, "w", wt->w, true, 16));
    if (wt->format == QMV_AFFINE) {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, true, tb));
        QMV_TRY(check_ptr(fn, "biases", wt->biases, true, tb));
    } else {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, true, scale_bytes(wt->format)));
    }
    QMV_TRY(check_ptr(fn, "global_scale", wt->global_scale, wt->global_scale != nullptr, 4));
    if (!library_scratch) QMV_TRY(check_ptr(fn, "workspace", workspace, true, 4));
    const size_t need = qmv_qvm_workspace_bytes(B, wt->K, wt->N);
    if (qmv::qvm_splits(B, wt->K, wt->N, nullptr) > 65535)
        return fail(QMV_ERR_UNSUPPORTED, "%s: N = %lld needs more than 65535 row splits at B = %lld",
                    fn, (long long)wt->N, (long long)B);
    if (library_scratch && need > qmv::kScratchBytes)
        return fail(QMV_ERR_UNSUPPORTED,
                    "%s: B = %lld, K = %lld, N = %lld needs %zu bytes of scratch; the library "
                    "holds %zu (call qmv_qvm with a workspace instead)", fn, (long long)B,
                    (long long)wt->K, (long long)wt->N, need, qmv::kScratchBytes);
    if (!library_scratch && workspace_bytes < need)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: workspace of %zu bytes, %zu needed", fn,
                    workspace_bytes, need);
    {
        const uintptr_t xs = (uintptr_t)x, xe = xs + (uintptr_t)(B * wt->N * tb);
        const uintptr_t ys = (uintptr_t)y, ye = ys + (uintptr_t)(B * wt->K * tb);
        if (xs < ye && ys < xe) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: x and y overlap", fn);
    }
    qmv::QvmParams q{};
    q.dtype = dtype; q.format = wt->format; q.bits = lp.bits; q.group = lp.group;
    q.B = B; q.K = wt->K; q.N = wt->N; q.row_bytes = lp.row_bytes; q.sc_per_row = lp.sc_per_row;
    q.x = x; q.w = wt->w; q.scales = wt->scales; q.biases = wt->biases;
    q.gscale = wt->format == QMV_NVFP4 ? wt->global_scale : nullptr;
    if (library_scratch) {
        if (const int e = qmv::scratch_for_current_device(&workspace))
            return fail(QMV_ERR_HIP, "%s: device scratch lookup failed: %s", fn,
                        qmv::hip_error_string(e));
    }
    q.y = y; q.ws = static_cast<float*>(workspace);
    q.splits = qmv::qvm_splits(q.B, q.K, q.N, &q.rows_per_split);
    return launch_status(qmv::launch_qvm(q, stream), fn);
}

qmv_status_t qmv_qvm(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* wt, int64_t B, const void* x,
                     void* y, void* workspace, size_t workspace_bytes) {
    return qvm_impl("qmv_qvm", stream, dtype, wt, B, x, y, workspace, workspace_bytes, false);
}

size_t qmv_qvm_noalloc_max_workspace_bytes(void) { return qmv::kScratchBytes; }

qmv_status_t qmv_qvm_noalloc(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* wt, int64_t B,
                             const void* x, void* y) {
    return qvm_impl("qmv_qvm_noalloc", stream, dtype, wt, B, x, y, nullptr, 0, true);
}

qmv_status_t qmv_rmsnorm_qmv(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* wt, int64_t B,
                             const void* x, const void* gamma, float eps, void* y) {
    const char* fn = "qmv_rmsnorm_qmv";
    if (wt == nullptr) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: weights struct is NULL", fn);
    if (wt->n_experts != 1)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: n_experts must be 1", fn);
    QMV_TRY(check_common(fn, dtype, B, wt->K, wt->N, 8));
    qmv::LaunchParams lp{};
    lp.dtype = dtype;
    QMV_TRY(format_geometry(fn, wt->format, wt->bits, wt->group_size, wt->K, lp));
    if (wt->format >= QMV_SB_E8M0)
        return fail(QMV_ERR_UNSUPPORTED, "%s: takes the affine, MXFP4, NVFP4 and MXFP8 formats",
                    fn);
    if (!(eps >= 0.0f) || eps > 3.0e38f)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
    if (B == 0 || wt->N == 0) return QMV_OK;
    const int tb = dtype_bytes(dtype);
    QMV_TRY(check_ptr(fn, "y", y, true, tb));
    if (wt->K == 0)   // empty sums
        return launch_status(qmv::launch_zero_fill(y, B * wt->N * tb, stream), fn);
    QMV_TRY(check_ptr(fn, "x", x, true, 16));
    QMV_TRY(check_ptr(fn, "gamma", gamma, true, 16));
    QMV_TRY(check_ptr(fn, "w", wt->w, true, 16));
    if (wt->format == QMV_AFFINE) {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, true, tb));
        QMV_TRY(check_ptr(fn, "biases", wt->biases, true, tb));
    } else {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, true, scale_bytes(wt->format)));
    }
    QMV_TRY(check_ptr(fn, "global_scale", wt->global_scale, wt->global_scale != nullptr, 4));
    {
        const uintptr_t xs = (uintptr_t)x, xe = xs + (uintptr_t)(B * wt->K * tb);
        const uintptr_t ys = (uintptr_t)y, ye = ys + (uintptr_t)(B * wt->N * tb);
        if (xs < ye && ys < xe) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: x and y overlap", fn);
        const uintptr_t gs = (uintptr_t)gamma, ge = gs + (uintptr_t)(wt->K * tb);
        if (gs < ye && ys < ge)
            return fail(QMV_ERR_INVALID_ARGUMENT, "%s: gamma and y overlap", fn);
    }
    lp.B = B; lp.K = wt->K; lp.N = wt->N;
    lp.x = x; lp.w = wt->w; lp.scales = wt->scales; lp.biases = wt->biases; lp.y = y;
    lp.gscale = wt->format == QMV_NVFP4 ? wt->global_scale : nullptr;
    qmv::NormArgs na{gamma, eps};
    return launch_status(qmv::launch_qmv_norm(lp, na, stream), fn);
}

size_t qmv_qmm_workspace_bytes(int64_t M, int64_t K, int64_t N, qmv_format_t format) {
    if (M <= 0 || K <= 0 || N <= 0) return 0;
    const int s = qmv::qmm_splits(M, K, N, format);
    return s > 1 ? (size_t)s * (size_t)M * (size_t)N * sizeof(float) : 0;
}

qmv_status_t qmv_qmm(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* wt, int64_t M, const void* x,
                     void* y, void* workspace, size_t workspace_bytes) {
    const char* fn = "qmv_qmm";
    if (wt == nullptr) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: weights struct is NULL", fn);
    if (wt->n_experts != 1)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: n_experts must be 1", fn);
    QMV_TRY(check_common(fn, dtype, 1, wt->K, wt->N, 1));
    if (dtype != QMV_BF16 && dtype != QMV_F16)
        return fail(QMV_ERR_UNSUPPORTED, "%s: activations must be bf16 or f16", fn);
    if (M < 0) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: M=%lld < 0", fn, (long long)M);
    if (M > (int64_t)65535 * 64)
        return fail(QMV_ERR_UNSUPPORTED, "%s: M=%lld above %d", fn, (long long)M, 65535 * 64);
    qmv::LaunchParams lp{};
    QMV_TRY(format_geometry(fn, wt->format, wt->bits, wt->group_size, wt->K, lp));
    if (wt->format >= QMV_SB_E8M0)
        return fail(QMV_ERR_UNSUPPORTED, "%s: qmm takes the affine, MXFP4, NVFP4 and MXFP8 "
                    "formats", fn);
    if (M == 0 || wt->N == 0) return QMV_OK;
    const int tb = dtype_bytes(dtype);
    QMV_TRY(check_ptr(fn, "y", y, true, tb));
    if (wt->K == 0)   // empty sums
        return launch_status(qmv::launch_zero_fill(y, M * wt->N * tb, stream), fn);
    QMV_TRY(check_ptr(fn, "x", x, true, 16));
    QMV_TRY(check_ptr(fn, "w", wt->w, true, 16));
    if (wt->format == QMV_AFFINE) {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, true, tb));
        QMV_TRY(check_ptr(fn, "biases", wt->biases, true, tb));
    } else {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, true, scale_bytes(wt->format)));
    }
    QMV_TRY(check_ptr(fn, "global_scale", wt->global_scale, wt->global_scale != nullptr, 4));
    {
        const uintptr_t xs = (uintptr_t)x, xe = xs + (uintptr_t)(M * wt->K * tb);
        const uintptr_t ys = (uintptr_t)y, ye = ys + (uintptr_t)(M * wt->N * tb);
        if (xs < ye && ys < xe) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: x and y overlap", fn);
    }
    const size_t need = qmv_qmm_workspace_bytes(M, wt->K, wt->N, wt->format);
    if (need > 0) {
        QMV_TRY(check_ptr(fn, "workspace", workspace, true, 4));
        if (workspace_bytes < need)
            return fail(QMV_ERR_INVALID_ARGUMENT, "%s: workspace of %zu bytes, %zu needed", fn,
                        workspace_bytes, need);
    }
    qmv::QmmParams q{};
    q.dtype = dtype; q.format = wt->format; q.bits = lp.bits; q.group = lp.group;
    q.M = M; q.N = wt->N; q.K = wt->K; q.row_bytes = lp.row_bytes; q.sc_per_row = lp.sc_per_row;
    q.x = x; q.w = wt->w; q.scales = wt->scales; q.biases = wt->biases;
    q.gscale = wt->format == QMV_NVFP4 ? wt->global_scale : nullptr;
    q.y = y;
    q.ws = static_cast<float*>(workspace);
    q.splits = qmv::qmm_splits(M, wt->K, wt->N, wt->format);
    return launch_status(qmv::launch_qmm(q, stream), fn);
}

qmv_status_t qmv_quantize_affine(hipStream_t stream, qmv_dtype_t dtype, int64_t N, int64_t K, const void* w,
                                 int bits, int group_size, uint8_t* packed, void* scales,
                                 void* biases) {
    return run_quantize("qmv_quantize_affine", stream, dtype, QMV_AFFINE, bits, group_size, N, K,
                        w, packed, scales, biases, nullptr);
}

qmv_status_t qmv_quantize_mxfp4(hipStream_t stream, qmv_dtype_t dtype, int64_t N, int64_t K, const void* w,
                                uint8_t* packed, uint8_t* scales) {
    return run_quantize("qmv_quantize_mxfp4", stream, dtype, QMV_MXFP4, 4, 32, N, K, w, packed,
                        scales, nullptr, nullptr);
}

qmv_status_t qmv_quantize_mxfp8(hipStream_t stream, qmv_dtype_t dtype, int64_t N, int64_t K, const void* w,
                                uint8_t* packed, uint8_t* scales) {
    return run_quantize("qmv_quantize_mxfp8", stream, dtype, QMV_MXFP8, 8, 32, N, K, w, packed,
                        scales, nullptr, nullptr);
}

qmv_status_t qmv_quantize_nvfp4(hipStream_t stream, qmv_dtype_t dtype, int64_t N, int64_t K, const void* w,
                                uint8_t* packed, uint8_t* scales, float* global_scale) {
    return run_quantize("qmv_quantize_nvfp4", stream, dtype, QMV_NVFP4, 4, 16, N, K, w, packed,
                        scales, nullptr, global_scale);
}

const char* qmv_last_error(void) { return g_last_error; }

qmv_status_t qmv_affine(hipStream_t stream, qmv_dtype_t dtype, int64_t B, int64_t K, int64_t N, const void* x,
                        const uint8_t* w, const void* scales, const void* biases, int bits,
                        int group_size, void* y) {
    return run_qmv("qmv_affine", stream, dtype, QMV_AFFINE, bits, group_size, B, K, N, x, w,
                   scales, biases, nullptr, y);
}

qmv_status_t qmv_fp_mxfp4(hipStream_t stream, qmv_dtype_t dtype, int64_t B, int64_t K, int64_t N,
                          const void* x, const uint8_t* w, const uint8_t* scales, void* y) {
    return run_qmv("qmv_fp_mxfp4", stream, dtype, QMV_MXFP4, 4, 32, B, K, N, x, w, scales,
                   nullptr, nullptr, y);
}

qmv_status_t qmv_fp_nvfp4(hipStream_t stream, qmv_dtype_t dtype, int64_t B, int64_t K, int64_t N,
                          const void* x, const uint8_t* w, const uint8_t* scales,
                          const float* global_scale, void* y) {
    return run_qmv("qmv_fp_nvfp4", stream, dtype, QMV_NVFP4, 4, 16, B, K, N, x, w, scales,
                   nullptr, global_scale, y);
}

qmv_status_t qmv_fp_block(hipStream_t stream, qmv_dtype_t dtype, qmv_format_t format,
                          qmv_element_t element, int block,
                          int64_t B, int64_t K, int64_t N, const void* x, const uint8_t* w,
                          const void* scales, void* y) {
    if (format < QMV_SB_E8M0 || format > QMV_SB_F16)
        return fail(QMV_ERR_INVALID_ARGUMENT, "qmv_fp_block: format %d is not a block-scaled "
                    "family (QMV_SB_E8M0 / QMV_SB_F32 / QMV_SB_F16)", format);
    return run_qmv("qmv_fp_block", stream, dtype, format, element, block, B, K, N, x, w, scales,
                   nullptr, nullptr, y);
}

qmv_status_t qmv_fp_mxfp8(hipStream_t stream, qmv_dtype_t dtype, int64_t B, int64_t K, int64_t N,
                          const void* x, const uint8_t* w, const uint8_t* scales, void* y) {
    return run_qmv("qmv_fp_mxfp8", stream, dtype, QMV_MXFP8, 8, 32, B, K, N, x, w, scales,
                   nullptr, nullptr, y);
}

qmv_status_t gather_qmv(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* wt, const void* x,
                        int64_t n_x_rows, const uint32_t* lhs_indices,
                        const uint32_t* rhs_indices, int64_t n_slots, void* y) {
    const char* fn = "gather_qmv";
    if (wt == nullptr) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: weights struct is NULL", fn);
    if (n_slots < 0 || n_x_rows < 0 || wt->n_experts < 0)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: negative count", fn);
    if (n_slots > ((int64_t)1 << 31) || wt->n_experts > 65534)
        return fail(QMV_ERR_UNSUPPORTED, "%s: n_slots or n_experts too large", fn);
    QMV_TRY(check_common(fn, dtype, 1, wt->K, wt->N, 1));
    qmv::LaunchParams lp{};
    lp.dtype = dtype;
    QMV_TRY(format_geometry(fn, wt->format, wt->bits, wt->group_size, wt->K, lp));
    if (wt->format >= QMV_SB_E8M0)
        return fail(QMV_ERR_UNSUPPORTED, "%s: the gather takes the affine, MXFP4, NVFP4 and "
                    "MXFP8 formats", fn);
    if (n_slots == 0 || wt->N == 0) return QMV_OK;
    const int tb = dtype_bytes(dtype);
    const bool has_w = wt->K > 0 && wt->n_experts > 0;
    QMV_TRY(check_ptr(fn, "y", y, true, tb));
    QMV_TRY(check_ptr(fn, "lhs_indices", lhs_indices, true, 4));
    QMV_TRY(check_ptr(fn, "rhs_indices", rhs_indices, true, 4));
    QMV_TRY(check_ptr(fn, "x", x, wt->K > 0 && n_x_rows > 0, 16));
    QMV_TRY(check_ptr(fn, "w", wt->w, has_w, 16));
    if (wt->format == QMV_AFFINE) {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, has_w, tb));
        QMV_TRY(check_ptr(fn, "biases", wt->biases, has_w, tb));
    } else {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, has_w, scale_bytes(wt->format)));
    }
    QMV_TRY(check_ptr(fn, "global_scale", wt->global_scale, wt->global_scale != nullptr, 4));
    lp.B = 1; lp.K = wt->K; lp.N = wt->N;
    lp.x = x; lp.w = wt->w; lp.scales = wt->scales; lp.biases = wt->biases;
    lp.gscale = wt->format == QMV_NVFP4 ? wt->global_scale : nullptr;
    lp.y = y;
    lp.n_experts = wt->n_experts; lp.n_x_rows = n_x_rows; lp.n_slots = n_slots;
    lp.lhs = lhs_indices; lp.rhs = rhs_indices;
    return launch_status(qmv::launch_gather(lp, stream), fn);
}

qmv_status_t gather_qmm(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* wt, const void* x,
                        int64_t n_x_rows, const uint32_t* lhs_indices,
                        const uint32_t* rhs_indices, int64_t n_slots, void* y) {
    const char* fn = "gather_qmm";
    if (wt == nullptr) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: weights struct is NULL", fn);
    if (n_slots < 0 || n_x_rows < 0 || wt->n_experts < 0)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: negative count", fn);
    if (n_slots > (int64_t)65535 * 64 || wt->n_experts > 65534)
        return fail(QMV_ERR_UNSUPPORTED, "%s: n_slots or n_experts too large", fn);
    QMV_TRY(check_common(fn, dtype, 1, wt->K, wt->N, 1));
    if (dtype != QMV_BF16 && dtype != QMV_F16)
        return fail(QMV_ERR_UNSUPPORTED, "%s: activations must be bf16 or f16", fn);
    qmv::LaunchParams lp{};
    QMV_TRY(format_geometry(fn, wt->format, wt->bits, wt->group_size, wt->K, lp));
    if (wt->format >= QMV_SB_E8M0)
        return fail(QMV_ERR_UNSUPPORTED, "%s: takes the affine, MXFP4, NVFP4 and MXFP8 formats",
                    fn);
    if (n_slots == 0 || wt->N == 0) return QMV_OK;
    const int tb = dtype_bytes(dtype);
    QMV_TRY(check_ptr(fn, "y", y, true, tb));
    if (wt->K == 0 || wt->n_experts == 0 || n_x_rows == 0)   // every row is empty or out of range
        return launch_status(qmv::launch_zero_fill(y, n_slots * wt->N * tb, stream), fn);
    QMV_TRY(check_ptr(fn, "lhs_indices", lhs_indices, true, 4));
    QMV_TRY(check_ptr(fn, "rhs_indices", rhs_indices, true, 4));
    QMV_TRY(check_ptr(fn, "x", x, true, 16));
    QMV_TRY(check_ptr(fn, "w", wt->w, true, 16));
    if (wt->format == QMV_AFFINE) {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, true, tb));
        QMV_TRY(check_ptr(fn, "biases", wt->biases, true, tb));
    } else {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, true, scale_bytes(wt->format)));
    }
    QMV_TRY(check_ptr(fn, "global_scale", wt->global_scale, wt->global_scale != nullptr, 4));
    {
        const uintptr_t xs = (uintptr_t)x, xe = xs + (uintptr_t)(n_x_rows * wt->K * tb);
        const uintptr_t ys = (uintptr_t)y, ye = ys + (uintptr_t)(n_slots * wt->N * tb);
        if (xs < ye && ys < xe) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: x and y overlap", fn);
    }
    qmv::QmmParams q{};
    q.dtype = dtype; q.format = wt->format; q.bits = lp.bits; q.group = lp.group;
    q.M = n_slots; q.N = wt->N; q.K = wt->K; q.row_bytes = lp.row_bytes;
    q.sc_per_row = lp.sc_per_row;
    q.x = x; q.w = wt->w; q.scales = wt->scales; q.biases = wt->biases;
    q.gscale = wt->format == QMV_NVFP4 ? wt->global_scale : nullptr;
    q.y = y;
    q.splits = 1;
    q.lhs = lhs_indices; q.rhs = rhs_indices;
    q.n_experts = wt->n_experts; q.n_x_rows = n_x_rows;
    // blocks per tile along z: about the distinct experts a tile of
    // consecutive slots sorted by expert holds (any count is correct: the
    // last one takes the rest)
    {
        const int64_t bm = qmv::qmm_block_rows(n_slots, wt->N, wt->format);
        int64_t runs = (wt->n_experts * bm + n_slots - 1) / n_slots + 1;
        if (runs > bm) runs = bm;
        if (runs > wt->n_experts) runs = wt->n_experts;
        if (runs > 64) runs = 64;
        q.runs = (int)(runs < 1 ? 1 : runs);
    }
    return launch_status(qmv::launch_qmm(q, stream), fn);
}

// ------------------------------- codecs ----------------------------------

int64_t qmv_packed_row_bytes(qmv_format_t format, int bits, int64_t K) {
    if (K < 0) return -1;
    switch (format) {
        case QMV_AFFINE:
            if (!valid_bits(bits) || (K * bits) % 8) return -1;
            return K * bits / 8;
        case QMV_MXFP4:
        case QMV_NVFP4:
            return K % 2 ? -1 : K / 2;
        case QMV_MXFP8:
            return K;
        default:
            return -1;
    }
}

qmv_status_t qmv_pack_codes(const uint8_t* codes, int64_t rows, int64_t K, int bits,
                            uint8_t* packed) {
    const char* fn = "qmv_pack_codes";
    if (!valid_bits(bits)) return fail(QMV_ERR_UNSUPPORTED, "%s: bits=%d", fn, bits);
    if (rows < 0 || K < 0 || (K * bits) % 8)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: bad shape rows=%lld K=%lld", fn,
                    (long long)rows, (long long)K);
    if (rows * K == 0) return QMV_OK;
    if (!codes || !packed) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
    const int64_t rb = K * bits / 8;
    const uint32_t lim = 1u << bits;
    for (int64_t i = 0; i < rows * K; ++i)
        if (codes[i] >= lim)
            return fail(QMV_ERR_INVALID_ARGUMENT, "%s: code %u at %lld does not fit %d bits", fn,
                        codes[i], (long long)i, bits);
    for (int64_t r = 0; r < rows; ++r) {
        uint8_t* out = packed + r * rb;
        memset(out, 0, (size_t)rb);
        const uint8_t* c = codes + r * K;
        // accumulate codes into a 64-bit window and flush whole bytes
        uint64_t acc = 0;
        int nacc = 0;
        int64_t o = 0;
        for (int64_t j = 0; j < K; ++j) {
            acc |= (uint64_t)c[j] << nacc;
            nacc += bits;
            while (nacc >= 8) {
                out[o++] = (uint8_t)(acc & 0xFF);
                acc >>= 8;
                nacc -= 8;
            }
        }
    }
    return QMV_OK;
}

qmv_status_t qmv_unpack_codes(const uint8_t* packed, int64_t rows, int64_t K, int bits,
                              uint8_t* codes) {
    const char* fn = "qmv_unpack_codes";
    if (!valid_bits(bits)) return fail(QMV_ERR_UNSUPPORTED, "%s: bits=%d", fn, bits);
    if (rows < 0 || K < 0 || (K * bits) % 8)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: bad shape", fn);
    if (rows * K == 0) return QMV_OK;
    if (!codes || !packed) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
    const int64_t rb = K * bits / 8;
    const uint32_t mask = (1u << bits) - 1u;
    for (int64_t r = 0; r < rows; ++r) {
        const uint8_t* in = packed + r * rb;
        uint64_t acc = 0;
        int nacc = 0;
        int64_t i = 0;
        for (int64_t j = 0; j < K; ++j) {
            while (nacc < bits) {
                acc |= (uint64_t)in[i++] << nacc;
                nacc += 8;
            }
            codes[r * K + j] = (uint8_t)(acc & mask);
            acc >>= bits;
            nacc -= bits;
        }
    }
    return QMV_OK;
}

qmv_status_t qmv_encode_e4m3(const float* v, int64_t n, uint8_t* out) {
    const char* fn = "qmv_encode_e4m3";
    if (n < 0) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: n < 0", fn);
    if (n == 0) return QMV_OK;
    if (!v || !out) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: NULL buffer", fn);
    for (int64_t i = 0; i < n; ++i) {
        const float f = v[i];
        if (isnan(f)) { out[i] = 0x7F; continue; }
        const uint8_t sign = signbit(f) ? 0x80 : 0x00;
        double a = fabs((double)f);
        if (a >= 448.0) { out[i] = sign | 0x7E; continue; }
        if (a == 0.0) { out[i] = sign; continue; }
        // a = m * 2^e with m in [1, 2); values below 2^-6 use the subnormal
        // spacing 2^-9
        int e2;
        frexp(a, &e2);
        int e = e2 - 1;
        if (e < -6) e = -6;
        const double step = ldexp(1.0, e - 3);         // 3 mantissa bits
        double q = a / step;                           // exact: power-of-two step
        double r = nearbyint(q);                       // ties to even (default mode)
        int64_t m = (int64_t)r;                        // 8..16 normal, 0..8 subnormal
        int code;
        if (e == -6 && m < 8) {
            code = (int)m;                             // subnormal: exponent field 0
        } else {
            if (m == 16) { m = 8; e += 1; }
            code = ((e + 7) << 3) | (int)(m - 8);
        }
        if (code > 0x7E) code = 0x7E;
        out[i] = sign | (uint8_t)code;
    }
    return QMV_OK;
}

qmv_status_t qmv_unpack_codes_device(hipStream_t stream, const uint8_t* packed, int64_t rows,
                                     int64_t K, int bits, uint8_t* codes) {
    const char* fn = "qmv_unpack_codes_device";
    if (!valid_bits(bits)) return fail(QMV_ERR_UNSUPPORTED, "%s: bits=%d", fn, bits);
    if (rows < 0 || K < 0 || K % 32)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: rows >= 0 and K %% 32 == 0 required", fn);
    if (rows * K == 0) return QMV_OK;
    QMV_TRY(check_ptr(fn, "packed", packed, true, 16));
    QMV_TRY(check_ptr(fn, "codes", codes, true, 1));
    return launch_status(qmv::launch_unpack_device(packed, rows, K, bits, codes, stream), fn);
}

qmv_status_t qmv_dequant_device(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* wt, float* out) {
    const char* fn = "qmv_dequant_device";
    if (wt == nullptr) return fail(QMV_ERR_INVALID_ARGUMENT, "%s: weights struct is NULL", fn);
    if (wt->n_experts != 1)
        return fail(QMV_ERR_INVALID_ARGUMENT, "%s: n_experts must be 1", fn);
    QMV_TRY(check_common(fn, dtype, 1, wt->K, wt->N, 1));
    qmv::LaunchParams lp{};
    lp.dtype = dtype;
    QMV_TRY(format_geometry(fn, wt->format, wt->bits, wt->group_size, wt->K, lp));
    if (wt->K == 0 || wt->N == 0) return QMV_OK;
    const int tb = dtype_bytes(dtype);
    QMV_TRY(check_ptr(fn, "w", wt->w, true, 16));
    QMV_TRY(check_ptr(fn, "out", out, true, 4));
    if (wt->format == QMV_AFFINE) {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, true, tb));
        QMV_TRY(check_ptr(fn, "biases", wt->biases, true, tb));
    } else {
        QMV_TRY(check_ptr(fn, "scales", wt->scales, true, scale_bytes(wt->format)));
    }
    QMV_TRY(check_ptr(fn, "global_scale", wt->global_scale, wt->global_scale != nullptr, 4));
    lp.B = 1; lp.K = wt->K; lp.N = wt->N;
    lp.w = wt->w; lp.scales = wt->scales; lp.biases = wt->biases;
    lp.gscale = wt->format == QMV_NVFP4 ? wt->global_scale : nullptr;
    return launch_status(qmv::launch_dequant_device(lp, out, stream), fn);
}

}  // extern "C"
