// Measurement kernels: a streaming read and a plain copy (see qmv_bench.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv_bench.h"

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Block b reads the 16-byte vectors [b*256*U, (b+1)*256*U): thread t loads
// vectors b*256*U + j*256 + t for j < U, all issued before any is used, so a
// lane keeps U*16 bytes in flight and every load instruction of a wave reads
// 1 KB of consecutive bytes.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const v4u* __restrict__ p, int64_t n,
                                                          uint32_t* __restrict__ sink) {
    const int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
    v4u v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int64_t i = base + (int64_t)j * 256;
        v[j] = __builtin_nontemporal_load(p + (i < n ? i : n - 1));
    }
    v4u a = v[0];
#pragma unroll
    for (int j = 1; j < U; ++j) a ^= v[j];
    const uint32_t r = a.x ^ a.y ^ a.z ^ a.w;
    // keep the loads live without a store per thread
    if (r == 0x9E3779B9u) sink[blockIdx.x & 0xFFFF] = r;
}

__global__ __launch_bounds__(256) void copy_kernel(const v4u* __restrict__ s, v4u* __restrict__ d,
                                                   int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        d[i] = s[i];
}

template <int U>
int launch_read(hipStream_t st, const v4u* p, int64_t n, uint32_t* sink) {
    const int64_t blocks = (n + 256 * U - 1) / (256 * U);
    if (blocks > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read_kernel<U>, dim3((unsigned)blocks), dim3(256), 0, st, p, n,
                       sink);
    return (int)hipGetLastError();
}

// One-shot read with T threads per block, U 16-byte loads per lane; with
// XCD the blocks run in XCD-contiguous order (block b of the 8-way
// round-robin dispatch takes the b/8-th range of XCD b % 8's share).
template <int T, int U, bool XCD>
__global__ __launch_bounds__(T) void read_oneshot_kernel(const v4u* __restrict__ p, int64_t n,
                                                         uint32_t* __restrict__ sink) {
    int64_t b = blockIdx.x;
    if (XCD) {
        const int64_t nb = gridDim.x, q = nb / 8, r = nb % 8, x = b % 8;
        b = x * q + (x < r ? x : r) + b / 8;
    }
    const int64_t base = b * T * U + threadIdx.x;
    v4u v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int64_t i = base + (int64_t)j * T;
        v[j] = __builtin_nontemporal_load(p + (i < n ? i : n - 1));
    }
    v4u a = v[0];
#pragma unroll
    for (int j = 1; j < U; ++j) a ^= v[j];
    const uint32_t r = a.x ^ a.y ^ a.z ^ a.w;
    if (r == 0x9E3779B9u) sink[blockIdx.x & 0xFFFF] = r;
}

// Each lane reads W consecutive 16-byte vectors (16 W bytes per lane).
template <int W>
__global__ __launch_bounds__(256) void read_wide_kernel(const v4u* __restrict__ p, int64_t n,
                                                        uint32_t* __restrict__ sink) {
    const int64_t base = ((int64_t)blockIdx.x * 256 + threadIdx.x) * W;
    v4u v[W];
#pragma unroll
    for (int j = 0; j < W; ++j) {
        const int64_t i = base + j;
        v[j] = __builtin_nontemporal_load(p + (i < n ? i : n - 1));
    }
    v4u a = v[0];
#pragma unroll
    for (int j = 1; j < W; ++j) a ^= v[j];
    const uint32_t r = a.x ^ a.y ^ a.z ^ a.w;
    if (r == 0x9E3779B9u) sink[blockIdx.x & 0xFFFF] = r;
}

// Persistent grid-stride read: a fixed grid, U loads per lane in flight per
// iteration; every lane runs the same number of iterations (clamped indices).
template <int U>
__global__ __launch_bounds__(256) void read_stride_kernel(const v4u* __restrict__ p, int64_t n,
                                                          uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t per_it = stride * U;
    const int64_t iters = (n + per_it - 1) / per_it;
    v4u a = {0u, 0u, 0u, 0u};
    for (int64_t it = 0; it < iters; ++it) {
        const int64_t base = it * per_it + (int64_t)blockIdx.x * 256 + threadIdx.x;
        v4u v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int64_t i = base + (int64_t)j * stride;
            v[j] = __builtin_nontemporal_load(p + (i < n ? i : n - 1));
        }
#pragma unroll
        for (int j = 0; j < U; ++j) a ^= v[j];
    }
    const uint32_t r = a.x ^ a.y ^ a.z ^ a.w;
    if (r == 0x9E3779B9u) sink[blockIdx.x & 0xFFFF] = r;
}

// Row patterns over [rows][2048 bytes] (the MXFP4 K=4096 row length): a wave
// reads 16 rows x 256 bytes with four instructions. MODE 0: eight lanes per
// 128-byte line (lane l: row l / 8 of an 8-row half, 16 bytes at l % 8);
// MODE 1: the 16x16x32 MFMA operand layout (lane l: row l % 16, 16 bytes at
// 16 (l / 16) of a 64-byte segment).
template <int MODE>
__global__ __launch_bounds__(256) void read_rows_kernel(const uint8_t* __restrict__ p,
                                                        int64_t rows, uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t r0 = (wv / 8) * 16;            // 8 waves across a row group's 2048 bytes
    const int64_t c0 = (wv % 8) * 256;
    v4u v[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        int64_t r;
        int64_t off;
        if (MODE == 0) {
            r = r0 + (s & 1) * 8 + lane / 8;
            off = c0 + 128 * (s >> 1) + 16 * (lane % 8);
        } else {
            r = r0 + lane % 16;
            off = c0 + 64 * s + 16 * (lane / 16);
        }
        r = r < rows ? r : rows - 1;
        v[s] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p + r * 2048 + off));
    }
    v4u a = v[0] ^ v[1] ^ v[2] ^ v[3];
    const uint32_t rr = a.x ^ a.y ^ a.z ^ a.w;
    if (rr == 0x9E3779B9u) sink[blockIdx.x & 0xFFFF] = rr;
}

// The one-row QMV's loads over [rows][2048] weight bytes followed by
// [rows][128] scale bytes (the MXFP4 K=4096 layout): a wave takes two rows;
// lane l reads 16 bytes at 16 l and 1024 + 16 l of each row, and scale bytes
// l and 64 + l of each row; four waves per block.
__global__ __launch_bounds__(256) void read_rowpair_kernel(const uint8_t* __restrict__ p,
                                                           int64_t rows,
                                                           uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2;
    const uint8_t* sc = p + rows * 2048;
    v4u a = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t r = r0 + i < rows ? r0 + i : rows - 1;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            a ^= __builtin_nontemporal_load(
                reinterpret_cast<const v4u*>(p + r * 2048 + 1024 * u + 16 * lane));
            a.x ^= __builtin_nontemporal_load(sc + r * 128 + 64 * u + lane);
        }
    }
    const uint32_t rr = a.x ^ a.y ^ a.z ^ a.w;
    if (rr == 0x9E3779B9u) sink[blockIdx.x & 0xFFFF] = rr;
}

// The one-row QMV's loads (as read_rowpair_kernel) followed by the write a
// QMV must make: each wave folds its 64 lanes' bytes (XOR across the wave, so
// every load is used) and lane 63 writes one 4-byte word per row pair, i.e.
// 2 bytes per row like a 16-bit y. With XCD, block b runs the row tile of the
// one-row QMV's XCD-chunked order (the eight blocks an XCD receives from each
// group of 64 own consecutive tiles).
template <bool XCD>
__global__ __launch_bounds__(256) void read_rowpair_write_kernel(const uint8_t* __restrict__ p,
                                                                 int64_t rows,
                                                                 uint32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    int64_t b = blockIdx.x;
    if (XCD) {
        const int64_t span = 64, grid = gridDim.x;
        if (b < (grid / span) * span) {
            const int64_t r = b % span;
            b = (b - r) + (r % 8) * 8 + r / 8;
        }
    }
    const int64_t r0 = (b * 4 + (threadIdx.x >> 6)) * 2;
    const uint8_t* sc = p + rows * 2048;
    v4u a = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t r = r0 + i < rows ? r0 + i : rows - 1;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            a ^= __builtin_nontemporal_load(
                reinterpret_cast<const v4u*>(p + r * 2048 + 1024 * u + 16 * lane));
            a.x ^= __builtin_nontemporal_load(sc + r * 128 + 64 * u + lane);
        }
    }
    uint32_t rr = a.x ^ a.y ^ a.z ^ a.w;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) rr ^= (uint32_t)__shfl_xor((int)rr, off);
    if (lane == 63 && r0 + 1 < rows) out[r0 / 2] = rr;
}

template <class Kern>
int launch_blocks(Kern k, int64_t blocks, int threads, hipStream_t st, const v4u* p, int64_t n,
                  uint32_t* sink) {
    if (blocks > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(threads), 0, st, p, n, sink);
    return (int)hipGetLastError();
}

}  // namespace

extern "C" int qmv_bench_read_design(void* stream, const void* buf, int64_t bytes,
                                     uint32_t* sink, int design) {
    if (bytes <= 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15))
        return (int)hipErrorInvalidValue;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const v4u* p = static_cast<const v4u*>(buf);
    const int64_t n = bytes / 16;
    auto nb = [&](int64_t per) { return (n + per - 1) / per; };
    switch (design) {
        case 0: return launch_blocks(read_oneshot_kernel<256, 2, false>, nb(512), 256, st, p, n, sink);
        case 1: return launch_blocks(read_oneshot_kernel<256, 4, false>, nb(1024), 256, st, p, n, sink);
        case 2: return launch_blocks(read_oneshot_kernel<256, 8, false>, nb(2048), 256, st, p, n, sink);
        case 3: return launch_blocks(read_oneshot_kernel<512, 4, false>, nb(2048), 512, st, p, n, sink);
        case 4: return launch_blocks(read_oneshot_kernel<1024, 2, false>, nb(2048), 1024, st, p, n, sink);
        case 5: return launch_blocks(read_oneshot_kernel<64, 8, false>, nb(512), 64, st, p, n, sink);
        case 6: return launch_blocks(read_oneshot_kernel<256, 4, true>, nb(1024), 256, st, p, n, sink);
        case 7: return launch_blocks(read_wide_kernel<2>, nb(512), 256, st, p, n, sink);
        case 8: return launch_blocks(read_wide_kernel<4>, nb(1024), 256, st, p, n, sink);
        case 9: return launch_blocks(read_stride_kernel<4>, 256, 256, st, p, n, sink);
        case 10: return launch_blocks(read_stride_kernel<4>, 512, 256, st, p, n, sink);
        case 11: return launch_blocks(read_stride_kernel<4>, 1024, 256, st, p, n, sink);
        case 12: return launch_blocks(read_stride_kernel<4>, 2048, 256, st, p, n, sink);
        case 13: return launch_blocks(read_stride_kernel<8>, 256, 256, st, p, n, sink);
        case 14: return launch_blocks(read_stride_kernel<8>, 512, 256, st, p, n, sink);
        case 15:
        case 16: {
            if (bytes % (2048 * 16)) return (int)hipErrorInvalidValue;
            const int64_t rows = bytes / 2048;
            auto* k = design == 15 ? read_rows_kernel<0> : read_rows_kernel<1>;
            // rows / 16 row groups x 8 waves, 4 waves per block
            hipLaunchKernelGGL(k, dim3((unsigned)(rows / 16 * 2)), dim3(256), 0, st,
                               static_cast<const uint8_t*>(buf), rows, sink);
            return (int)hipGetLastError();
        }
        case 17: {
            if (bytes % (2176 * 8)) return (int)hipErrorInvalidValue;
            const int64_t rows = bytes / 2176;   // 2048 weight + 128 scale bytes per row
            hipLaunchKernelGGL(read_rowpair_kernel, dim3((unsigned)(rows / 8)), dim3(256), 0, st,
                               static_cast<const uint8_t*>(buf), rows, sink);
            return (int)hipGetLastError();
        }
        case 18:
        case 19: {
            // as 17, plus a 2-byte-per-row write to sink (65536 words: rows <= 131072)
            if (bytes % (2176 * 8)) return (int)hipErrorInvalidValue;
            const int64_t rows = bytes / 2176;
            if (rows > 2 * 65536) return (int)hipErrorInvalidValue;
            auto* k = design == 18 ? read_rowpair_write_kernel<false>
                                   : read_rowpair_write_kernel<true>;
            hipLaunchKernelGGL(k, dim3((unsigned)(rows / 8)), dim3(256), 0, st,
                               static_cast<const uint8_t*>(buf), rows, sink);
            return (int)hipGetLastError();
        }
        default: return (int)hipErrorInvalidValue;
    }
}

extern "C" int qmv_bench_stream_read(void* stream, const void* buf, int64_t bytes,
                                     uint32_t* sink, int unroll) {
    if (bytes < 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15))
        return (int)hipErrorInvalidValue;
    if (bytes == 0) return 0;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const v4u* p = static_cast<const v4u*>(buf);
    const int64_t n = bytes / 16;
    switch (unroll) {
        case 1: return launch_read<1>(st, p, n, sink);
        case 2: return launch_read<2>(st, p, n, sink);
        case 4: return launch_read<4>(st, p, n, sink);
        case 8: return launch_read<8>(st, p, n, sink);
        case 16: return launch_read<16>(st, p, n, sink);
        default: return (int)hipErrorInvalidValue;
    }
}

extern "C" int qmv_bench_copy(void* stream, const void* src, void* dst, int64_t bytes) {
    if (bytes < 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15) ||
        (reinterpret_cast<uintptr_t>(dst) & 15))
        return (int)hipErrorInvalidValue;
    if (bytes == 0) return 0;
    const int64_t n = bytes / 16;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const v4u*>(src),
                       static_cast<v4u*>(dst), n);
    return (int)hipGetLastError();
}
