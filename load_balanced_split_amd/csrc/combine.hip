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
// One workgroup of 256 threads per (segment, query head of its group).
// Pass 1 reduces M and sum w over the chunks' LSEs; pass 2 streams the
// normalised partial rows with float4 loads, D/4 threads per row and
// 256 / (D/4) rows in flight per round, then reduces the rows in LDS.
#include "common.h"

namespace hpcattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr float kNegInf = -__builtin_inff();

__device__ float block_reduce(float v, bool is_max, float *s_red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float x = __shfl_xor(v, o, 64);
        v = is_max ? fmaxf(v, x) : v + x;
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s_red[w] = v;
    __syncthreads();
    float r = s_red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = is_max ? fmaxf(r, s_red[i]) : r + s_red[i];
    __syncthreads();
    return r;
}

template <int D>
__global__ void __launch_bounds__(kThreads) combine_kernel(CombineParams p) {
    constexpr int kRowThreads = D / 4;                 // float4 per partial row
    constexpr int kRows = kThreads / kRowThreads;      // rows per round
    __shared__ float s_red[kThreads / 64];
    __shared__ f32x4 s_acc[kRows][kRowThreads];

    const int64_t s = blockIdx.x;
    const int g = blockIdx.y;
    const int G = p.G;
    int64_t k0, k1;
    if (p.seg_off) {
        k0 = p.seg_off[s];
        k1 = p.seg_off[s + 1];
    } else {
        k0 = s * p.stride;
        k1 = k0 + p.stride;
    }
    const int64_t n = k1 - k0;

    float mx = kNegInf;
    for (int64_t k = threadIdx.x; k < n; k += kThreads) mx = fmaxf(mx, p.part_lse[(k0 + k) * G + g]);
    const float M = block_reduce(mx, true, s_red);
    const int64_t out_row = s * G + g;
    bf16x2 *out = reinterpret_cast<bf16x2 *>(reinterpret_cast<__bf16 *>(p.out) + out_row * D);
    if (M == kNegInf) {   // no live KV: out = 0, lse = -inf
        for (int i = threadIdx.x; i < D / 2; i += kThreads) out[i] = bf16x2{(__bf16)0.f, (__bf16)0.f};
        if (p.out_lse && threadIdx.x == 0) p.out_lse[out_row] = kNegInf;
        return;
    }
    float ws = 0.f;
    for (int64_t k = threadIdx.x; k < n; k += kThreads) {
        const float l = p.part_lse[(k0 + k) * G + g];
        ws += l == kNegInf ? 0.f : __expf(l - M);
    }
    const float wsum = block_reduce(ws, false, s_red);

    const int row = threadIdx.x / kRowThreads, c4 = threadIdx.x % kRowThreads;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int64_t k = row;
#pragma unroll 4
    for (; k < n; k += kRows) {
        const float l = p.part_lse[(k0 + k) * G + g];
        if (l == kNegInf) continue;   // an empty split: no weight, row never written
        const f32x4 o = *reinterpret_cast<const f32x4 *>(p.part_o + ((k0 + k) * G + g) * D + 4 * c4);
        acc += __expf(l - M) * o;
    }
    s_acc[row][c4] = acc;
    __syncthreads();
    if (row == 0) {
        for (int i = 1; i < kRows; ++i) acc += s_acc[i][c4];
        acc = acc * (1.0f / wsum);
        out[2 * c4] = bf16x2{(__bf16)acc[0], (__bf16)acc[1]};
        out[2 * c4 + 1] = bf16x2{(__bf16)acc[2], (__bf16)acc[3]};
        if (p.out_lse && c4 == 0) p.out_lse[out_row] = M + __logf(wsum);
    }
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
