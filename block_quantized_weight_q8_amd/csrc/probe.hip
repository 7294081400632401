// Pure-read probe and cache flush for the measurements (see q8gemv_probe.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemv_device.hpp"
#include "q8gemv_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = Q8G_PROBE_SINK_WORDS;

// NT: nontemporal (streaming) loads, as the GEMV weights; otherwise plain cached
// loads, as the activations (the two calibrate the hardware read counters)
template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_kernel(const int4 *__restrict__ src, int64_t n16,
                                                         uint32_t *__restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    uint32_t acc = 0;
    constexpr int U = 8;
    // U strided loads in flight per thread in every round, the last round too: indexes
    // past the end re-read the last element (cached) and are left out of the digest
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += U * stride) {
        int4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + u * stride;
            const int4 *p = src + (j < n16 ? j : n16 - 1);
            v[u] = NT ? q8g::load16_stream(p) : q8g::load16(p);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i + u * stride < n16) acc ^= (uint32_t)(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
    }
    // one digest word per block, written by a vector store from lane 0
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    __shared__ uint32_t part[kThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kThreads / 64; ++w) t ^= part[w];
        sink[blockIdx.x] = t;
    }
}

__global__ __launch_bounds__(kThreads) void flush_kernel(int4 *__restrict__ buf, int64_t n16, uint32_t value)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int v = (int)value;
    const int4 w = {v, v, v, v};
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) buf[i] = w;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

q8g_status probe(bool nt, const void *src, int64_t bytes, uint32_t *sink, void *stream)
{
    if (bytes < 0 || bytes % 16) return Q8G_ERR_SHAPE;
    if (!src || !sink) return Q8G_ERR_NULL;
    if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3)) return Q8G_ERR_ALIGN;
    const int4 *s = static_cast<const int4 *>(src);
    int64_t n16 = bytes / 16;
    uint32_t *k = sink;
    void *args[] = {&s, &n16, &k};
    // about eight 16-byte loads per thread, so that a small buffer is read by a grid
    // of its own size (the same shape as a GEMV launch over it), at most kBlocks
    int64_t blocks = (n16 + kThreads * 8 - 1) / (kThreads * 8);
    blocks = blocks < 1 ? 1 : blocks > kBlocks ? kBlocks : blocks;
    const void *fn = nt ? reinterpret_cast<const void *>(&probe_kernel<true>)
                        : reinterpret_cast<const void *>(&probe_kernel<false>);
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, 0,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}

}  // namespace

extern "C" {

q8g_status q8g_probe_read(const void *src, int64_t bytes, uint32_t *sink, void *stream)
{
    return probe(true, src, bytes, sink, stream);
}

q8g_status q8g_probe_read_cached(const void *src, int64_t bytes, uint32_t *sink, void *stream)
{
    return probe(false, src, bytes, sink, stream);
}

q8g_status q8g_flush(void *buf, int64_t bytes, uint32_t value, void *stream)
{
    if (bytes < 0 || bytes % 16) return Q8G_ERR_SHAPE;
    if (bytes == 0) return Q8G_OK;
    if (!buf) return Q8G_ERR_NULL;
    if (!aligned16(buf)) return Q8G_ERR_ALIGN;
    int4 *b = static_cast<int4 *>(buf);
    int64_t n16 = bytes / 16;
    uint32_t v = value;
    void *args[] = {&b, &n16, &v};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&flush_kernel), dim3(4096),
                                         dim3(kThreads), args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}

}  // extern "C"
