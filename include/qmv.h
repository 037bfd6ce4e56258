/*
 * qmv.h - C ABI of the MI355X (gfx950) quantized matrix-vector product library.
 *
 * Computes the decode-time quantized matrix-vector product
 *
 *     y[b, n] = sum_k x[b, k] * dequant(W)[n, k]      0 <= b < B <= 8
 *
 * over packed low-bit weights, in four weight formats:
 *
 *   affine  2/3/4/5/6/8-bit unsigned codes q, one scale s and one bias beta per
 *           group of 32/64/128 consecutive k: w = s*q + beta ("wh-iron
 *           kernel-op coverage audit", section "Quantization precision
 *           coverage", Track 2; "mlx 1.0.0 - quantized_nax.h", `dequantize`).
 *           The bias term is beta * sum(x) with every x widened to fp32 before
 *           it is added ("ml-explore/mlx pull request 4516", description).
 *   MXFP4   E2M1 elements, one E8M0 power-of-two scale per block of 32.
 *   NVFP4   E2M1 elements, one E4M3 scale per block of 16, one fp32 global.
 *   MXFP8   E4M3 elements, one E8M0 scale per block of 32.
 *           (the three block-scaled formats: the same audit's Track-1 table).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers of the compute calls are DEVICE pointers to row-major,
 *   contiguous data. The caller owns all memory; nothing here allocates.
 * - `stream` is a hipStream_t (NULL = the default stream). Compute calls are
 *   asynchronous on it and never synchronize. `dtype` is a qmv_dtype_t;
 *   values outside the enum are rejected (QMV_ERR_INVALID_ARGUMENT).
 * - x, y and the affine scales/biases share one element type `dtype`
 *   (f32, f16 or bf16); y is written in that type, rounded to nearest-even
 *   from an fp32 accumulation.
 * - Packed weight rows: code j of a row sits at bits [j*b, (j+1)*b) of the
 *   row's little-endian bit stream (LSB first; for 4-bit codes the even k is
 *   the low nibble; 8-bit codes are bytes). Row bytes = K*b/8.
 * - E4M3 is the OCP "fn" variant (bias 7, max 448, NaN only at 0x7F/0xFF,
 *   no infinity). E8M0 byte e means 2^(e-127); e = 255 is NaN.
 * - Requirements checked before any HIP call (a failed check returns an
 *   error, leaves every output untouched and records a message):
 *     B in [0, 8]; K >= 0, K % 32 == 0 (affine: also K % group == 0);
 *     N >= 0; K <= 2^24 and N <= 2^28 (else QMV_ERR_UNSUPPORTED);
 *     bits in {2,3,4,5,6,8}; group in {32,64,128};
 *     w and x 16-byte aligned, y / scales / biases aligned to their element;
 *     pointers may be NULL only where the tensor is empty.
 *   B == 0 or N == 0 is a successful no-op. K == 0 writes y = 0.
 * - x and y must not overlap.
 * - Errors: every entry point returns a qmv_status_t; qmv_last_error()
 *   gives the message of the last failure on the calling thread. A launch
 *   failure reported by the HIP runtime maps to QMV_ERR_HIP (asynchronous
 *   faults surface at the caller's next synchronization, as with any kernel).
 * - Thread safety: the state is a thread-local error message and, per kernel
 *   and device, the largest dynamic LDS size already requested from the HIP
 *   runtime (raised under a lock). Calls from several threads are safe.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { QMV_F32 = 0, QMV_F16 = 1, QMV_BF16 = 2 } qmv_dtype_t;

typedef enum {
    QMV_AFFINE = 0, QMV_MXFP4 = 1, QMV_NVFP4 = 2, QMV_MXFP8 = 3,
    /* symmetric block-scaled family, by scale storage (qmv_fp_block; in
     * qmv_weights_t: bits = the element code, group_size = the block) */
    QMV_SB_E8M0 = 4, QMV_SB_F32 = 5, QMV_SB_F16 = 6
} qmv_format_t;

/* Elements of the symmetric block-scaled family: OCP E2M1 / E4M3 (fn) / E5M2
 * micro-floats, or two's-complement integers of n bits (QMV_EL_INT + n). */
typedef enum { QMV_EL_E2M1 = 1, QMV_EL_E4M3 = 2, QMV_EL_E5M2 = 3, QMV_EL_INT = 10 } qmv_element_t;

typedef enum {
    QMV_OK = 0,
    QMV_ERR_INVALID_ARGUMENT = 1,
    QMV_ERR_UNSUPPORTED = 2,
    QMV_ERR_MISALIGNED = 3,
    QMV_ERR_HIP = 4
} qmv_status_t;

/* Affine QMV ("mlx 1.0.0 - quantized_nax.h": `qdot`, whose per-group result is
 * scale * sum(x*q) + bias * sum(x); the fp32 widening of sum(x) follows
 * "ml-explore/mlx pull request 4516").
 *   x      [B, K]           dtype
 *   w      [N, K*bits/8]    uint8, packed codes
 *   scales [N, K/group]     dtype
 *   biases [N, K/group]     dtype
 *   y      [B, N]           dtype (output)
 * Output rows are independent: the result for row n does not depend on N,
 * so a call with N not a multiple of any tile gives, for rows < N, the same
 * bits as a padded call ("ml-explore/mlx pull request 4516", Correctness). */
qmv_status_t qmv_affine(hipStream_t stream, qmv_dtype_t dtype, int64_t B, int64_t K, int64_t N,
                        const void* x, const uint8_t* w, const void* scales,
                        const void* biases, int bits, int group_size, void* y);

/* MXFP4 QMV.  w [N, K/2] uint8 (E2M1 codes, even k in the low nibble),
 * scales [N, K/32] uint8 (E8M0). x [B, K], y [B, N] in dtype. */
qmv_status_t qmv_fp_mxfp4(hipStream_t stream, qmv_dtype_t dtype, int64_t B, int64_t K, int64_t N,
                          const void* x, const uint8_t* w, const uint8_t* scales, void* y);

/* NVFP4 QMV.  w [N, K/2] uint8 (E2M1), scales [N, K/16] uint8 (E4M3),
 * global_scale: DEVICE pointer to one fp32, or NULL for 1.0; it multiplies
 * each fp32 row sum once ("ml-explore/mlx pull request 4516": NVFP4 calls with
 * a global scale). K % 32 == 0 is required (two scale blocks per 32 codes). */
qmv_status_t qmv_fp_nvfp4(hipStream_t stream, qmv_dtype_t dtype, int64_t B, int64_t K, int64_t N,
                          const void* x, const uint8_t* w, const uint8_t* scales,
                          const float* global_scale, void* y);

/* Symmetric block-scaled QMV: the rest of the Track-1 format matrix ("wh-iron
 * kernel-op coverage audit", "Quantization precision coverage": element x
 * block x scale storage, no zero point). w [N, K*bits/8] packed codes (LSB
 * first; 8-bit codes are bytes), scales [N, K/block] of the format's storage:
 *   format         element             block    name on the page
 *   QMV_SB_E8M0    E5M2                32       mxfp8_e5m2
 *   QMV_SB_E8M0    int2..int8          32       mxint2..mxint8
 *   QMV_SB_F32     E4M3                16       nvfp8
 *   QMV_SB_F32     E2M1 / E4M3 / E5M2  32       fp4 / fp8_e4m3 / fp8_e5m2
 *   QMV_SB_F32     int2..int8          64       int2..int8
 *   QMV_SB_F16     as QMV_SB_F32                the *_f16 twins
 * Value of a code: element(code) * scale of its block; an mxint element is
 * read as fixed point with one integer bit, code * 2^-(n-2) (OCP MXINT8's
 * reading, which the audit extends to the other widths). E5M2 is OCP's (bias
 * 15; exponent 31 holds infinity and NaN). Other (element, block, format)
 * combinations are QMV_ERR_UNSUPPORTED; K % block == 0. Alignment: scales to
 * their element (1, 4 or 2 bytes). fp32 accumulation; each unit of 32 codes
 * folds one scale per 16-code half. */
qmv_status_t qmv_fp_block(hipStream_t stream, qmv_dtype_t dtype, qmv_format_t format,
                          qmv_element_t element, int block,
                          int64_t B, int64_t K, int64_t N, const void* x, const uint8_t* w,
                          const void* scales, void* y);

/* MXFP8 (E4M3 elements) QMV.  w [N, K] uint8 (E4M3), scales [N, K/32] uint8
 * (E8M0). x [B, K], y [B, N] in dtype. */
qmv_status_t qmv_fp_mxfp8(hipStream_t stream, qmv_dtype_t dtype, int64_t B, int64_t K, int64_t N,
                          const void* x, const uint8_t* w, const uint8_t* scales, void* y);

/* Expert-stacked quantized weights for gather_qmv. Expert e's N x K matrix
 * starts at w + e*N*row_bytes, its scales at scales + e*N*(K/block) (and the
 * affine biases likewise), block = group_size (affine), 32 (MX) or 16 (NV).
 * `bits` and `group_size` are read for QMV_AFFINE only; `global_scale`
 * (device fp32 or NULL) for QMV_NVFP4 only and is shared by all experts. */
typedef struct {
    qmv_format_t format;
    int bits;
    int group_size;
    int64_t n_experts;
    int64_t N;
    int64_t K;
    const uint8_t* w;
    const void* scales;      /* dtype (affine) or uint8 (block-scaled) */
    const void* biases;      /* affine only */
    const float* global_scale;
} qmv_weights_t;

/* Routed-expert gathered QMV ("mlx 1.0.0 - quantized_nax.h",
 * `adjust_matrix_offsets` with lhs/rhs indices; "@lgrammel/ds4-provider -
 * moe.metal", `kernel_mul_mv_id`):
 *     y[s, :] = W[rhs_indices[s]] . x[lhs_indices[s], :]     0 <= s < n_slots
 *   x [n_x_rows, K] dtype; indices uint32 [n_slots] (device); y [n_slots, N].
 * Each expert's weights are read once per call however many slots use it.
 * An index out of range (expert >= n_experts or x row >= n_x_rows) yields a
 * row of zeros ("ferrum-kernels - primitives.rs" tests: out-of-range ids give
 * zeros, not a fault). Each slot's row equals, bit for bit, a one-row
 * qmv_* call on that expert and x row. `w` points to host memory (the struct
 * itself); the pointers inside it are device pointers. */
qmv_status_t gather_qmv(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* w, const void* x,
                        int64_t n_x_rows, const uint32_t* lhs_indices,
                        const uint32_t* rhs_indices, int64_t n_slots, void* y);

/* Routed-expert gathered qmm: the gather_qmv product for many slots at once,
 * on the matrix cores (the MoE prefill form: "mlx 1.0.0 - quantized_nax.h",
 * `affine_gather_qmm_rhs_nax`, whose expert indices are sorted so that runs
 * of rows share an expert; "@lgrammel/ds4-provider - moe.metal",
 * `kernel_mul_mm_id`). Same arguments, semantics and out-of-range rule as
 * gather_qmv; dtype QMV_BF16 or QMV_F16 (QMV_F32 returns
 * QMV_ERR_UNSUPPORTED); n_slots <= 65535 * 64. Arithmetic as in qmv_qmm
 * (weights enter the MFMAs as dtype: exact for MXFP4 / NVFP4 / MXFP8 in bf16;
 * affine per group in fp32). A block of 64 or 128 consecutive slots runs its
 * K loop once per distinct expert among them, so rhs_indices sorted by expert
 * (runs of equal ids) is the fast order; any order is correct. Within such a
 * block the other experts' slots take zero x rows, so the weights must be
 * finite (an infinite or NaN weight of one expert would turn those rows into
 * NaN). */
qmv_status_t gather_qmm(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* w, const void* x,
                        int64_t n_x_rows, const uint32_t* lhs_indices,
                        const uint32_t* rhs_indices, int64_t n_slots, void* y);

/* ---------------- codecs: HOST memory, synchronous, no GPU needed -------- */

/* Bytes of one packed row: K*bits/8 for QMV_AFFINE, K/2 for the fp4 formats,
 * K for MXFP8 ("mlx 1.0.0 - quantized_nax.h", `get_pack_factor` /
 * `get_bytes_per_pack`). Returns -1 for invalid arguments. */
int64_t qmv_packed_row_bytes(qmv_format_t format, int bits, int64_t K);

/* Pack codes [rows, K] (uint8, each < 2^bits) into rows of K*bits/8 bytes,
 * LSB first: code j at bits [j*bits, (j+1)*bits) of the row's little-endian
 * bit stream ("wh-iron kernel-op coverage audit", "Quantization precision
 * coverage", Track 1: sub-byte codes packed tightly, least significant bit
 * first; the per-width masks of `dequantize` in "mlx 1.0.0 -
 * quantized_nax.h" read this layout). HOST pointers; codes [rows, K] and
 * packed [rows, K*bits/8] are caller-owned. Requires bits in {2,3,4,5,6,8}
 * and K*bits % 8 == 0 (QMV_ERR_INVALID_ARGUMENT / QMV_ERR_UNSUPPORTED
 * otherwise); a code >= 2^bits is QMV_ERR_INVALID_ARGUMENT, found before
 * anything is written, so packed is left untouched. */
qmv_status_t qmv_pack_codes(const uint8_t* codes, int64_t rows, int64_t K, int bits,
                            uint8_t* packed);

/* Inverse of qmv_pack_codes (same layout and passages): packed [rows,
 * K*bits/8] -> codes [rows, K], HOST pointers, caller-owned. Same argument
 * checks as qmv_pack_codes. */
qmv_status_t qmv_unpack_codes(const uint8_t* packed, int64_t rows, int64_t K, int bits,
                              uint8_t* codes);

/* fp32 -> E4M3 (fn) bytes, for building NVFP4 block scales (the E4M3 block
 * scale of the NVFP4 row of the "wh-iron kernel-op coverage audit" Track-1
 * table; the E4M3 constants of its kv_cache op row: 3 mantissa bits, largest
 * value 448, a NaN sentinel). Round to nearest, ties to even; magnitudes
 * above 448 (and infinities) saturate to +-448; NaN gives 0x7F; the sign of
 * zero is kept. v [n] fp32 and out [n] bytes are HOST pointers, caller-owned;
 * NULL with n > 0 or n < 0 is QMV_ERR_INVALID_ARGUMENT. */
qmv_status_t qmv_encode_e4m3(const float* v, int64_t n, uint8_t* out);

/* ---------------- codecs: DEVICE memory, asynchronous ---------------------
 * These run the same decode functions as the QMV kernels, so their bit-exact
 * agreement with the definitions covers the hot path's decode. */

/* Device unpack: codes [rows, K] uint8 from packed rows [rows, K*bits/8]
 * (DEVICE pointers, caller-owned; asynchronous on stream), the layout of
 * qmv_pack_codes (audit Track 1, LSB first; "mlx 1.0.0 - quantized_nax.h"
 * `dequantize` masks), through the kernels' own code extraction. Same
 * argument checks as qmv_pack_codes, before any HIP call; a failed launch is
 * QMV_ERR_HIP. */
qmv_status_t qmv_unpack_codes_device(hipStream_t stream, const uint8_t* packed, int64_t rows,
                                     int64_t K, int bits, uint8_t* codes);

/* Device dequant of one matrix (w->n_experts must be 1) to fp32 [N, K]
 * (DEVICE out, caller-owned; asynchronous on stream): affine fmaf(s, q, beta)
 * (`dequantize` of "mlx 1.0.0 - quantized_nax.h": scale * q + bias); MXFP4
 * e2m1*2^(e-127); NVFP4 (e2m1*e4m3)*global; MXFP8 e4m3*2^(e-127) (the
 * element and scale definitions of the "wh-iron kernel-op coverage audit"
 * Track-1 table). Each value is the fp32 rounding of the exact one.
 * `dtype` is the storage type of the affine scales/biases (ignored
 * otherwise). The weight arguments are checked as for gather_qmv before any
 * HIP call; a failed launch is QMV_ERR_HIP. */
qmv_status_t qmv_dequant_device(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* w, float* out);

/* ---------------- qvm: DEVICE, asynchronous ---------------------------------
 * The transposed product y[b, k] = sum_n x[b, n] * dequant(W)[n, k] over the
 * same packed weights ("mlx 1.0.0 - quantized_nax.h", `qouter`: row n adds
 * x[n] * (scale * q + bias) across its columns). w: one matrix
 * (n_experts = 1) of the affine, MXFP4, NVFP4 or MXFP8 format, N rows of K
 * codes; x [B, N], y [B, K] in dtype, 1 <= B <= 8 (B = 0 is a no-op).
 * workspace: caller-owned device memory of at least
 * qmv_qvm_workspace_bytes(B, K, N) bytes (4-byte aligned), which the call
 * overwrites: row splits write fp32 partial sums there and a second kernel
 * adds them in split order, so repeated calls give identical results. Calls
 * that share a workspace must not overlap. N == 0 writes y = 0. A split holds
 * at most 8192 / B rows and a launch at most 65535 splits, so N above
 * 65535 * 8192 / B returns QMV_ERR_UNSUPPORTED. */
size_t qmv_qvm_workspace_bytes(int64_t B, int64_t K, int64_t N);
qmv_status_t qmv_qvm(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* w, int64_t B, const void* x,
                     void* y, void* workspace, size_t workspace_bytes);

/* qvm without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. Same arguments, kernels and
 * results as qmv_qvm (bit for bit), but the fp32 split partials go to a
 * library-held device scratch of qmv_qvm_noalloc_max_workspace_bytes() bytes
 * (16 MiB; one copy per device, held until the process ends, its address
 * looked up once per device on the first call there). A problem whose
 * qmv_qvm_workspace_bytes(B, K, N) exceeds that returns QMV_ERR_UNSUPPORTED
 * before any HIP call. Every call on a device shares that device's scratch:
 * calls that overlap on one device (two streams, or two threads) race and
 * must be serialized by the caller. The scratch keeps the last call's
 * partials; each call overwrites every element it reads, so nothing needs
 * clearing. Calls nothing that allocates (no hipMalloc / hipFree). */
size_t qmv_qvm_noalloc_max_workspace_bytes(void);
qmv_status_t qmv_qvm_noalloc(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* w, int64_t B,
                             const void* x, void* y);

/* ---------------- fused RMSNorm + QMV: DEVICE memory, asynchronous ----------
 * y[b, :] = W . (x[b, :] * r[b] * gamma) with r[b] = 1 / sqrt(mean_k x[b, k]^2
 * + eps) ("wh-iron kernel-op coverage audit", op rows "rms_norm" and
 * "rms_norm_qgemv (RMSNorm + quantized GEMV fused)", and the block-scaled
 * family's "fused RMSNorm + GEMV"), in one dispatch. r is one scalar per row,
 * so it multiplies the fp32 dot products before the final rounding; the
 * matrix-vector step reads RN_T(x[b, k] * gamma[k]) (the product of two T
 * values is exact in fp32, so this is one rounding). r is formed in fp32
 * (squares summed in fp32 in a fixed order, correctly rounded division and
 * square root). w: one matrix of the affine, MXFP4, NVFP4 or MXFP8 formats
 * (n_experts == 1); x [B, K] and gamma [K] in dtype (16-byte aligned);
 * y [B, N]; 1 <= B <= 8 (B = 0 is a no-op); eps finite and >= 0. K == 0 writes
 * y = 0. */
qmv_status_t qmv_rmsnorm_qmv(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* w, int64_t B,
                             const void* x, const void* gamma, float eps, void* y);

/* ---------------- qmm (batched product): DEVICE memory, asynchronous ---------
 * y[m, n] = sum_k x[m, k] * W[n, k] for M rows of activations at once (the
 * transposed qmm of "mlx 1.0.0 - quantized_nax.h": activations against the
 * packed [N, K] matrix the QMV entry points read; "wh-iron kernel-op coverage
 * audit", op row "quantized (affine_qmv / qvm / qmm)": the M-batched prefill
 * product), for batches past the QMV's eight rows. w: one matrix
 * (n_experts == 1) of the affine, MXFP4, NVFP4 or MXFP8 formats; x [M, K]
 * (16-byte aligned) and y [M, N] in dtype, which must be QMV_BF16 or QMV_F16
 * (QMV_F32 returns QMV_ERR_UNSUPPORTED); 0 <= M <= 65535 * 64 (M == 0 or
 * N == 0 is a no-op, K == 0 writes y = 0). Products run on the matrix cores
 * with fp32 accumulation: MXFP4 / MXFP8 / NVFP4 weights enter them as
 * code * block scale rounded to dtype, which is exact in bf16 (and in f16
 * while the value lies in f16's normal range); affine codes enter as integers
 * and scale and bias are applied per group in fp32 (s * sum x q + b * sum x);
 * NVFP4's global scale multiplies the fp32 result; y is rounded to dtype once.
 * workspace: caller-owned device memory of qmv_qmm_workspace_bytes(M, K, N, format)
 * bytes (4-byte aligned; may be NULL when that is 0). When M and N give too
 * few output tiles to fill the GPU, K is split over blocks that write fp32
 * partial sums there and a second kernel adds them in split order, so
 * repeated calls give identical results; calls that share a workspace must
 * not overlap. */
size_t qmv_qmm_workspace_bytes(int64_t M, int64_t K, int64_t N, qmv_format_t format);
qmv_status_t qmv_qmm(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* w, int64_t M, const void* x,
                     void* y, void* workspace, size_t workspace_bytes);

/* ---------------- fused routed-MoE decode block: DEVICE, asynchronous -------
 * The decode step of a routed mixture-of-experts FFN in two calls
 * ("@lgrammel/ds4-provider - moe.metal": the fused gate/up + activation
 * kernel and the per-token down kernel over its expert slots; "wh-iron
 * kernel-op coverage audit", op row "moe routed-expert decode fuse": two
 * dispatches, router weights folded in the down step). Slot s = t * top_k + j
 * of token t uses expert expert_ids[s] (uint32, [n_tokens, top_k]); a slot
 * whose id is >= n_experts gives a zero mid row and adds nothing to y. */

/* mid[s, :] = silu(g) * u in T, with g = gate[e] . x[t], u = up[e] . x[t]
 * (fp32 accumulation as in qmv_*), each clamped first when clamp > 1e-6
 * (g = min(g, clamp), u = clamp(u, -clamp, clamp)); silu(g) = g / (1 + exp(-g)).
 * gate and up: same format / bits / group / n_experts / N (= ffn) / K
 * (= hidden); x [n_tokens, K] (16-byte aligned); mid [n_tokens * top_k, N].
 * Requires 2 * K * sizeof(T) <= 64 KB. */
qmv_status_t qmv_moe_gate_up_swiglu(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* gate,
                                    const qmv_weights_t* up, const void* x, int64_t n_tokens,
                                    const uint32_t* expert_ids, int64_t top_k, float clamp,
                                    void* mid);

/* y[t, :] = sum_j route_weights[t, j] * (down[e] . mid[t * top_k + j, :]),
 * accumulated in fp32 and rounded to T once. down: N = hidden, K = ffn;
 * mid [n_tokens * top_k, K] in T (16-byte aligned); route_weights fp32
 * [n_tokens, top_k]; y [n_tokens, N]. Requires top_k <= 16,
 * top_k * K * sizeof(T) <= 64 KB and n_tokens <= 65535. Expert weights are read
 * per token, so repeated experts across tokens are served from cache. */
qmv_status_t qmv_moe_down_reduce(hipStream_t stream, qmv_dtype_t dtype, const qmv_weights_t* down,
                                 const void* mid, int64_t n_tokens, const uint32_t* expert_ids,
                                 const float* route_weights, int64_t top_k, void* y);

/* ---------------- quantize from float: DEVICE memory, asynchronous ---------
 * Encode a row-major [N, K] matrix w of `dtype` values (16-byte aligned) into
 * the layout the QMV entry points read: packed rows [N, row_bytes] (16-byte
 * aligned) and block scales. The pages ("wh-iron kernel-op coverage audit",
 * "Quantization precision coverage": Track 2's min/max encoder, the
 * fp_quantized / kv_cache rows' max-scale rounding, the Track-1 NVFP4 layout)
 * leave steps open; the readings below fix them. Every step that decides a
 * code is one fp32 operation in the order written (round to nearest even,
 * correctly rounded division), so the output is defined bit for bit. Inputs
 * must be finite. N == 0 or K == 0 is a successful no-op. K % 32 == 0 (affine:
 * also K % group_size == 0); K <= 2^24. Outputs must not overlap w. */

/* Affine, per group of group_size along K: lo, hi = group min, max (zero
 * extremes count as +0);
 * s32 = (hi - lo) / (2^bits - 1); scales = RN_T(s32), biases = RN_T(lo)
 * ([N, K/group_size], in dtype); q = clamp(rint((w - b) / s), 0, 2^bits - 1)
 * against the stored s and b, or 0 where the stored s is 0. */
qmv_status_t qmv_quantize_affine(hipStream_t stream, qmv_dtype_t dtype, int64_t N, int64_t K, const void* w,
                                 int bits, int group_size, uint8_t* packed, void* scales,
                                 void* biases);

/* MXFP4 / MXFP8, per block of 32: a = max |w|; scale byte (E8M0) = 0 if
 * a == 0, else clamp(floor(log2 a) - emax + 127, 0, 254) with emax 2 (E2M1)
 * or 8 (E4M3); element = nearest E2M1 / E4M3 to w / 2^(byte - 127), ties to
 * even, saturating at 6 / 448, sign kept (so -0 encodes with the sign bit).
 * scales [N, K/32] bytes. */
qmv_status_t qmv_quantize_mxfp4(hipStream_t stream, qmv_dtype_t dtype, int64_t N, int64_t K, const void* w,
                                uint8_t* packed, uint8_t* scales);
qmv_status_t qmv_quantize_mxfp8(hipStream_t stream, qmv_dtype_t dtype, int64_t N, int64_t K, const void* w,
                                uint8_t* packed, uint8_t* scales);

/* NVFP4: global = A / 2688 with A = max |w| over the matrix (written to the
 * device fp32 *global_scale, which is also used as the reduction's working
 * word while the call runs); per block of 16: sb = (max |w| / 6) / global,
 * scale byte = nearest E4M3 to sb (saturating); d = decoded scale * global;
 * element = nearest E2M1 to w / d, or code 0 where d is 0. scales [N, K/16]. */
qmv_status_t qmv_quantize_nvfp4(hipStream_t stream, qmv_dtype_t dtype, int64_t N, int64_t K, const void* w,
                                uint8_t* packed, uint8_t* scales, float* global_scale);

/* Message for the last non-OK status returned on this thread ("" if none):
 * every entry point returns a typed status and records a readable message
 * with it (the typed error results with a message of "ferrum-kernels 0.8.0 -
 * primitives.rs"). The string is owned by the library and stays valid until
 * the thread's next failing call. */
const char* qmv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
