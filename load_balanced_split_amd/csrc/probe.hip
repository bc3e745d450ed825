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

}  // namespace

hipError_t launch_stream_read(const void *buf, size_t bytes, int32_t workgroups, int32_t flags,
                              uint32_t *sink, hipStream_t stream) {
    const int64_t n = (int64_t)(bytes / 16);
    if (flags & 1)
        hipLaunchKernelGGL(stream_read_kernel<true>, dim3(workgroups), dim3(kProbeThreads), 0,
                           stream, reinterpret_cast<const u32x4 *>(buf), n, sink);
    else
        hipLaunchKernelGGL(stream_read_kernel<false>, dim3(workgroups), dim3(kProbeThreads), 0,
                           stream, reinterpret_cast<const u32x4 *>(buf), n, sink);
    return hipGetLastError();
}

}  // namespace hpcattn
