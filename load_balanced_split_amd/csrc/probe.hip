// A plain streaming read of a device buffer: the achievable HBM read
// bandwidth on this GPU, the measured reference next to the 8 TB/s spec.
//
// Each thread reads 16-byte vectors (plain or nontemporal loads) in a
// grid-stride loop, eight loads in flight per round, and folds them with XOR; the result is stored only if it
// equals a sentinel, which keeps every load live without writing traffic.
#include "common.h"

namespace hpcattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kUnroll = 8;

template <bool kNontemporal>
__global__ void __launch_bounds__(kProbeThreads)
stream_read_kernel(const u32x4 *__restrict__ p, int64_t n, uint32_t *sink) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = kNontemporal ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n; i += stride) acc ^= p[i];
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == 0x9E3779B9u) sink[0] = x;
}

// The same bytes read as 16 KB chunks in a scattered order: chunk c of the
// grid-stride sequence is physical chunk (c * odd) mod n, a bijection when n
// is a power of two.  This is the access shape of the decode kernel, which
// reads shuffled 16 KB (page, head) tiles.
template <bool kNontemporal>
__global__ void __launch_bounds__(kProbeThreads)
chunk_read_kernel(const u32x4 *__restrict__ p, int64_t nchunks, uint32_t *sink) {
    constexpr int kVecPerChunk = 16384 / 16;
    constexpr int kPerThread = kVecPerChunk / kProbeThreads;   // 4
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t c = blockIdx.x; c < nchunks; c += 2 * (int64_t)gridDim.x) {
        const int64_t c2 = c + gridDim.x < nchunks ? c + gridDim.x : c;
        const u32x4 *a = p + ((c * 0x9E3779B1ll) & (nchunks - 1)) * kVecPerChunk;
        const u32x4 *b = p + ((c2 * 0x9E3779B1ll) & (nchunks - 1)) * kVecPerChunk;
        u32x4 v[2 * kPerThread];
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const int i = u * kProbeThreads + threadIdx.x;
            v[u] = kNontemporal ? __builtin_nontemporal_load(a + i) : a[i];
            v[kPerThread + u] = kNontemporal ? __builtin_nontemporal_load(b + i) : b[i];
        }
#pragma unroll
        for (int u = 0; u < 2 * kPerThread; ++u) acc ^= v[u];
    }
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace

hipError_t launch_stream_read(const void *buf, size_t bytes, int32_t workgroups, int32_t flags,
                              uint32_t *sink, hipStream_t stream) {
    const int64_t n = (int64_t)(bytes / 16);
    if (flags & 2) {
        const int64_t nchunks = (int64_t)(bytes / 16384);
        if (flags & 1)
            hipLaunchKernelGGL(chunk_read_kernel<true>, dim3(workgroups), dim3(kProbeThreads), 0,
                               stream, reinterpret_cast<const u32x4 *>(buf), nchunks, sink);
        else
            hipLaunchKernelGGL(chunk_read_kernel<false>, dim3(workgroups), dim3(kProbeThreads), 0,
                               stream, reinterpret_cast<const u32x4 *>(buf), nchunks, sink);
        return hipGetLastError();
    }
    if (flags & 1)
        hipLaunchKernelGGL(stream_read_kernel<true>, dim3(workgroups), dim3(kProbeThreads), 0,
                           stream, reinterpret_cast<const u32x4 *>(buf), n, sink);
    else
        hipLaunchKernelGGL(stream_read_kernel<false>, dim3(workgroups), dim3(kProbeThreads), 0,
                           stream, reinterpret_cast<const u32x4 *>(buf), n, sink);
    return hipGetLastError();
}

}  // namespace hpcattn
