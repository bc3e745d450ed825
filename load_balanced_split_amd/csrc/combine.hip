// The combine step: merge each (request, KV head) segment's partials under
// the global softmax.
//
// "HPC-Ops x SGLang", section "Scheduling around live KV work": since each
// persistent workgroup produces only some of a request's partials, a final
// kernel reads the actual chunk count of every request and head and merges
// the partials under the correct global softmax normalisation.  "Hy3 preview
// full-stack inference optimization", section 2.1.1: a Combine kernel merges
// the split-KV results.
//
//   M = max_k lse_k,  w_k = exp(lse_k - M),
//   out = sum_k w_k o_k / sum_k w_k,  out_lse = M + ln sum_k w_k.
//
// One workgroup of 4 waves per (segment, query head of its group).  Wave w
// merges chunks w, w + 4, ... in one pass with a running maximum (each lane
// owns D/64 consecutive elements of the row, so a chunk's row is one
// coalesced 512-byte read), four chunks' loads in flight per wave; the four
// waves are then merged in LDS.  A chunk with lse = -inf (an empty static
// split) carries no weight and its row is never read.
#include "common.h"

namespace hpcattn {
namespace {


constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;
constexpr float kNegInf = -__builtin_inff();

// Running log-sum-exp merge state of one wave lane: max M, weight sum W and
// the weighted row `acc` (both relative to M).
template <int E>
struct Merge {
    float M = kNegInf, W = 0.f;
    float acc[E] = {};
    __device__ void add(float l, const float (&o)[E]) {
        if (l == kNegInf) return;
        const float M2 = fmaxf(M, l);
        const float a = __expf(M - M2), c = __expf(l - M2);   // M = -inf gives a = 0
        W = W * a + c;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = acc[e] * a + c * o[e];
        M = M2;
    }
};

template <int D>
__global__ void __launch_bounds__(kThreads) combine_kernel(CombineParams p) {
    constexpr int E = D / 64;   // elements per lane
    __shared__ float s_m[kWaves], s_w[kWaves];
    __shared__ float s_acc[kWaves][D];

    const int64_t s = blockIdx.x;
    const int g = blockIdx.y;
    const int G = p.G;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int64_t k0, k1;
    if (p.seg_off) {
        k0 = p.seg_off[s];
        k1 = p.seg_off[s + 1];
    } else {
        k0 = s * p.stride;
        k1 = k0 + p.stride;
    }
    const int64_t n = k1 - k0;

    Merge<E> mg;
    for (int64_t k = w; k < n; k += kWaves * kUnroll) {
        float l[kUnroll];
        float o[kUnroll][E];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t kk = k + u * kWaves;
            const int64_t row = (k0 + (kk < n ? kk : k)) * G + g;
            l[u] = kk < n ? p.part_lse[row] : kNegInf;
            const float *src = p.part_o + row * D + lane * E;
#pragma unroll
            for (int e = 0; e < E; ++e) o[u][e] = l[u] == kNegInf ? 0.f : src[e];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) mg.add(l[u], o[u]);
    }
    if (lane == 0) {
        s_m[w] = mg.M;
        s_w[w] = mg.W;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) s_acc[w][lane * E + e] = mg.acc[e];
    __syncthreads();
    if (w != 0) return;

    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) M = fmaxf(M, s_m[i]);
    const int64_t out_row = s * G + g;
    __bf16 *out = reinterpret_cast<__bf16 *>(p.out) + out_row * D + lane * E;
    if (M == kNegInf) {   // no live KV: out = 0, lse = -inf
#pragma unroll
        for (int e = 0; e < E; ++e) out[e] = (__bf16)0.f;
        if (p.out_lse && lane == 0) p.out_lse[out_row] = kNegInf;
        return;
    }
    float W = 0.f, acc[E] = {};
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const float c = s_m[i] == kNegInf ? 0.f : __expf(s_m[i] - M);
        W += c * s_w[i];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += c * s_acc[i][lane * E + e];
    }
    const float inv = 1.0f / W;
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = (__bf16)(acc[e] * inv);
    if (p.out_lse && lane == 0) p.out_lse[out_row] = M + __logf(W);
}

}  // namespace

hipError_t launch_combine(const CombineParams &p, hipStream_t stream) {
    if (p.S <= 0) return hipSuccess;
    const dim3 grid((unsigned)p.S, (unsigned)p.G);
    if (p.D == 128)
        hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hpcattn
