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

}  // namespace

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
