// Internal declarations shared by the host API and the HIP kernels.
// Not part of the public ABI (that is include/qmv.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace qmv {

enum Dtype { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum Format {
    FMT_AFFINE = 0, FMT_MXFP4 = 1, FMT_NVFP4 = 2, FMT_MXFP8 = 3,
    // symmetric block-scaled family, by scale storage; the element is the
    // "bits" field (an Element code) and the block length the "group" field
    FMT_SB_E8M0 = 4, FMT_SB_F32 = 5, FMT_SB_F16 = 6
};
// Element codes of the symmetric block-scaled family: micro-floats, or
// two's-complement integers of width n (code 10 + n).
enum Element { EL_E2M1 = 1, EL_E4M3 = 2, EL_E5M2 = 3, EL_INT = 10 };
constexpr int element_bits(int el) {
    return el == EL_E2M1 ? 4 : (el <= EL_E5M2 ? 8 : el - EL_INT);
}

// Everything one launch needs. Filled and validated by the host API.
struct LaunchParams {
    int dtype;          // Dtype of x, y and affine scales/biases
    int format;         // Format
    int bits;           // affine code width (4 for fp4, 8 for fp8)
    int group;          // affine group size (scale block for the others)
    int64_t B;          // batch rows (qmv) ; unused by gather
    int64_t K, N;
    int64_t row_bytes;  // packed bytes per weight row
    int64_t sc_per_row; // scale entries per weight row
    const void* x;
    const uint8_t* w;
    const void* scales;
    const void* biases;
    const float* gscale;
    void* y;
    // gather only
    int64_t n_experts, n_x_rows, n_slots;
    const uint32_t* lhs;
    const uint32_t* rhs;
};

// Extra arguments of the fused routed-MoE kernels, kept out of LaunchParams:
// every byte of kernel arguments costs scalar registers, and the QMV kernel
// sits at the scalar-register limit. The up matrix of the gate/up pair (same
// format and shape as w), slots per token (x row of slot s = s / top_k), the
// activation clamp (off when <= 1e-6) and the router weights [T, top_k].
struct MoeArgs {
    const uint8_t* w2;
    const void* scales2;
    const void* biases2;
    const float* gscale2;
    int64_t top_k;
    float act_clamp;
    const float* route_w;
};
struct NoMoeArgs {};

// Fused RMSNorm in front of a QMV: gamma [K] in T (16-byte aligned), eps >= 0.
struct NormArgs {
    const void* gamma;
    float eps;
};
int launch_qmv_norm(const LaunchParams& p, const NormArgs& na, void* stream);

int launch_moe_gate_up(const LaunchParams& p, const MoeArgs& m, void* stream);
int launch_zero_fill(void* p, int64_t bytes, void* stream);   // bytes % 2 == 0
int launch_moe_down(const LaunchParams& p, const MoeArgs& m, void* stream);

// One qvm call: y[B, K] = x[B, N] . W[N, K] (W packed as for QMV). Row splits
// write fp32 partials to ws ([splits, B, K]); a second pass adds them.
struct QvmParams {
    int dtype;
    int format;
    int bits;
    int group;
    int64_t B, K, N;
    int64_t row_bytes, sc_per_row;
    const void* x;
    const uint8_t* w;
    const void* scales;
    const void* biases;
    const float* gscale;
    void* y;
    float* ws;
    int64_t rows_per_split;
    int splits;
};
int launch_qvm(const QvmParams& q, void* stream);
// Output columns per qvm block: a lane owns a whole 32-code unit for B <= 2,
// 8 columns of one for larger B (8 accumulators per batch row).
inline int64_t qvm_tile_cols(int64_t B) { return B <= 2 ? 2048 : 512; }

// Row splits of a qvm launch: about 224 blocks of 8 waves (B <= 2) or 512
// blocks of 4 waves (B > 2) over the column tiles, each split between 64 * B
// rows (a batch of 8 rows per wave at least, and fp32 partials a small
// fraction of the weight bytes) and 8192 / B rows (its x rows fit 32 KB of LDS
// as fp32); depends on B, K and N alone.
inline int qvm_splits(int64_t B, int64_t K, int64_t N, int64_t* rows_per_split) {
    const int64_t bb = B < 1 ? 1 : B;
    const int64_t tc = qvm_tile_cols(bb);
    const int64_t tiles = (K + tc - 1) / tc;
    const int64_t target = bb <= 2 ? 224 : 512;
    int64_t s = tiles > 0 ? (target + tiles - 1) / tiles : 1;
    const int64_t lo = (N + 64 * bb - 1) / (64 * bb);     // splits at >= 64 B rows
    const int64_t hi_rows = 8192 / bb;
    const int64_t need = (N + hi_rows - 1) / hi_rows;     // splits at <= 8192 / B rows
    if (s > lo) s = lo;
    if (s < need) s = need;
    if (s < 1) s = 1;
    const int64_t rps = N > 0 ? (N + s - 1) / s : 1;
    if (rows_per_split) *rows_per_split = rps;
    return N > 0 ? (int)((N + rps - 1) / rps) : 1;
}

// One qmm call: y[M, N] = x[M, K] . W[N, K]^T (W packed as for QMV), 16-bit
// activations on the matrix cores.
struct QmmParams {
    int dtype;
    int format;
    int bits;
    int group;
    int64_t M, N, K;
    int64_t row_bytes, sc_per_row;
    const void* x;
    const uint8_t* w;
    const void* scales;
    const void* biases;
    const float* gscale;
    void* y;
    float* ws;    // [splits, M, N] fp32 partials when splits > 1
    int splits;   // K slices split over blocks (1 = none)
    // gather (rhs != nullptr): M = slots, x row lhs[s], expert rhs[s] of
    // n_experts stacked matrices; splits must be 1
    const uint32_t* lhs;
    const uint32_t* rhs;
    int64_t n_experts;
    int64_t n_x_rows;
    int runs;     // gather: blocks per tile along z (the last takes any further experts)
};
int launch_qmm(const QmmParams& q, void* stream);
// Rows of a qmm block tile: 128 when 128-row tiles alone give at least 256
// tiles (one per compute unit), else 64 (affine codes: always 64, their group
// accumulators would double the registers).
inline int qmm_block_rows(int64_t M, int64_t N, int format) {
    const int64_t tiles128 = ((M + 127) / 128) * ((N + 127) / 128);
    return format != 0 && M > 64 && tiles128 >= 256 ? 128 : 64;
}
// K splits of a qmm launch: none once the output tiles (block rows x 128)
// reach 256 (one per compute unit); else enough to reach about 512 blocks, at
// most 8 and with at least 8 slices of 64 codes each. Depends on M, K, N and
// the format.
inline int qmm_splits(int64_t M, int64_t K, int64_t N, int format) {
    const int64_t bm = qmm_block_rows(M, N, format);
    const int64_t tiles = ((N + 127) / 128) * ((M + bm - 1) / bm);
    const int64_t nk = (K + 63) / 64;
    if (tiles <= 0 || tiles >= 256) return 1;
    int64_t s = (512 + tiles - 1) / tiles;
    if (s > 8) s = 8;
    if (s > nk / 8) s = nk / 8;
    if (s < 1) return 1;
    const int64_t per = (nk + s - 1) / s;   // slices per split; no split is empty
    return (int)((nk + per - 1) / per);
}

// One quantize-from-float call: w [N, K] in `dtype` to the packed format.
struct QuantParams {
    int dtype;
    int format;
    int bits;            // affine code width
    int group;           // affine group size
    int64_t N, K;
    const void* w;
    uint8_t* packed;
    void* scales;        // T for affine, bytes for the block-scaled formats
    void* biases;        // affine only
    float* global_scale; // NVFP4 only: written (device fp32)
};

// Launchers (defined in the .hip translation units). Return 0 on success or
// the hipError_t of a failed launch.
int launch_quantize(const QuantParams& q, void* stream);
int launch_qmv(const LaunchParams& p, void* stream);
int launch_gather(const LaunchParams& p, void* stream);
int launch_unpack_device(const uint8_t* packed, int64_t rows, int64_t K, int bits,
                         uint8_t* codes, void* stream);
int launch_dequant_device(const LaunchParams& p, float* out, void* stream);
const char* hip_error_string(int err);

// Largest LDS footprint of the x staging buffer, in bytes.
constexpr int kMaxStageBytes = 64 * 1024;

// Size of the library-held device scratch of the entry points that allocate
// nothing (one copy per device, held until the process ends).
constexpr size_t kScratchBytes = (size_t)16 << 20;
// Device address of that scratch on the current device (looked up once per
// device and recorded). Returns 0 or a hipError_t.
int scratch_for_current_device(void** out);

}  // namespace qmv
