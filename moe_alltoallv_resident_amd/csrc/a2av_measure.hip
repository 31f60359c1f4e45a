// Measurement kernels (not on the path): plain one-direction streams, the read-only and
// write-only bandwidth this GPU reaches.  A kernel that reads r bytes and writes w bytes
// cannot beat (r + w) / (r / read_bw + w / write_bw); bench.py reports every path
// kernel against that mixed ceiling next to the nominal HBM peak.
#include "../../include/a2av.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;       // 16-byte vectors per thread in flight

// Read-only stream: every 16-byte vector of src read once (non-temporal, kUnroll in flight
// per thread, issued at clamped indices and masked), folded by XOR into one word per
// thread, written to out[thread].  The XOR of all out words is the XOR of all src words.
__global__ void __launch_bounds__(kThreads) read_stream_kernel(const u32x4* __restrict__ src, uint32_t* __restrict__ out,
                                                               int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
    uint32_t acc = 0;
    for (int64_t i0 = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; i0 < n; i0 += stride) {
        u32x4 r[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = i0 + (int64_t)u * kThreads;
            r[u] = __builtin_nontemporal_load(src + (i < n ? i : n - 1));
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = i0 + (int64_t)u * kThreads;
            const uint32_t m = i < n ? 0xFFFFFFFFu : 0u;
            acc ^= (r[u][0] ^ r[u][1] ^ r[u][2] ^ r[u][3]) & m;
        }
    }
    out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// Write-only stream: vector i of dst gets {i, i >> 32, 0x5A5A5A5A, ~i} (cacheable stores:
// measured a little faster than non-temporal ones for a pure write stream).
__global__ void __launch_bounds__(kThreads) write_stream_kernel(u32x4* __restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
    for (int64_t i0 = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; i0 < n; i0 += stride) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = i0 + (int64_t)u * kThreads;
            if (i < n) dst[i] = u32x4{(uint32_t)i, (uint32_t)((uint64_t)i >> 32), 0x5A5A5A5Au, ~(uint32_t)i};
        }
    }
}

}  // namespace

extern "C" int a2av_stream_reference(const void* src, void* dst, int64_t bytes, int32_t mode, void* stream) {
    if (bytes < 0 || bytes % 16 != 0) return A2AV_ERR_INVALID;
    if (mode != A2AV_STREAM_READ && mode != A2AV_STREAM_WRITE) return A2AV_ERR_INVALID;
    if (!dst || ((uintptr_t)dst % 16) != 0) return A2AV_ERR_INVALID;
    if (mode == A2AV_STREAM_READ && bytes > 0 && (!src || ((uintptr_t)src % 16) != 0)) return A2AV_ERR_INVALID;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return A2AV_ERR_HIP;
    const int64_t n = bytes / 16;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (mode == A2AV_STREAM_READ) {
        // four blocks per CU (measured best for a read stream), never more than the
        // output holds
        const int64_t max_blocks = A2AV_STREAM_READ_OUT_BYTES / (4 * kThreads);
        const unsigned grid = (unsigned)(4 * (int64_t)cus < max_blocks ? 4 * (int64_t)cus : max_blocks);
        if (n == 0) return A2AV_OK;
        hipLaunchKernelGGL(read_stream_kernel, dim3(grid), dim3(kThreads), 0, st, (const u32x4*)src, (uint32_t*)dst, n);
    } else {
        if (n == 0) return A2AV_OK;
        hipLaunchKernelGGL(write_stream_kernel, dim3((unsigned)(16 * cus)), dim3(kThreads), 0, st, (u32x4*)dst, n);
    }
    return hipGetLastError() == hipSuccess ? A2AV_OK : A2AV_ERR_HIP;
}
