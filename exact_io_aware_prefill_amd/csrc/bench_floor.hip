// Measurement helpers (declared in include/attn_bench.h): the floors a split-KV
// decode call is measured against.  Not part of the attention path.
//   * attn_bench_stream_read: one kernel that reads two device buffers of the same
//     size once (the decode's K and V caches) with 16-byte loads, grid-stride, on
//     a given number of 256-thread workgroups; each wave stores one word (the XOR
//     of what it read) so nothing is dead code.  Its time is what a plain read of
//     the decode's bytes costs at that grid, launch included.
//   * attn_bench_empty: an empty kernel of one workgroup, launched after the read
//     to time the cost of a second, dependent launch (the decode's combine).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_bench.h"

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;  // 16-byte loads in flight per lane

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4 *a, const uint4 *b, size_t n16,
                                                               uint32_t *sink)
{
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (int buf = 0; buf < 2; ++buf) {
        const uint4 *p = buf ? b : a;
        size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
        for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
            uint4 v[kInFlight];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) v[u] = p[i + u * stride];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
        for (; i < n16; i += stride) {
            const uint4 v = p[i];
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0) sink[(size_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" {

int attn_bench_stream_read(const void *a, const void *b, size_t bytes_each, int workgroups, uint32_t *sink,
                           void *stream)
{
    if (!a || !b || !sink) return -1;
    if (workgroups <= 0 || bytes_each % 16 != 0 || (reinterpret_cast<uintptr_t>(a) & 15u) ||
        (reinterpret_cast<uintptr_t>(b) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u))
        return -2;
    if (bytes_each == 0) return 0;
    (void)hipGetLastError();
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4 *>(a), static_cast<const uint4 *>(b),
                       bytes_each / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

int attn_bench_empty(void *stream)
{
    (void)hipGetLastError();
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
