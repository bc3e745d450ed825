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
// With R query rows per request (draft verify), a segment's partials hold
// R G rows each, row r G + g for query row r and head h G + g, and every row
// is merged on its own.
//
// A workgroup of 4 waves merges 4 / WPR rows of one segment, WPR waves per
// row.  Wave k of a row merges chunks k, k + WPR, ... in one pass with a
// running maximum (each lane owns D/64 consecutive elements of the row, so a
// chunk's row is one coalesced read), U chunks' loads in flight per wave;
// with WPR > 1 the row's waves are then merged in LDS.  WPR = 4 suits
// segments cut into many chunks (a long request over many bins; U = 16, so
// 64 chunks take one round of loads), WPR = 1 segments of a few chunks with
// many rows (U = 4).  A chunk with lse = -inf (an empty static split, whose
// O row is never written) carries no weight: its row is loaded with the
// others, so that no load waits for another, but never enters the sums.
#include "common.h"

namespace hpcattn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kNegInf = -__builtin_inff();

// Chunks in flight per wave.
template <int WPR>
constexpr int unroll() {
    return WPR > 1 ? 16 : 4;
}

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

template <int D, int WPR>
__global__ void __launch_bounds__(kThreads) combine_kernel(CombineParams p) {
    constexpr int E = D / 64;            // elements per lane
    constexpr int RPW = kWaves / WPR;    // rows per workgroup
    __shared__ float s_m[kWaves], s_w[kWaves];
    __shared__ float s_acc[kWaves][D];

    const int64_t s = blockIdx.x;
    const int G = p.G, RG = p.R * p.G;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = blockIdx.y * RPW + w / WPR;   // partial row r G + g
    const int part = w % WPR;
    int64_t k0, k1;
    if (p.seg_off) {
        k0 = p.seg_off[s];
        k1 = p.seg_off[s + 1];
    } else {
        k0 = s * p.stride;
        k1 = k0 + p.stride;
    }
    const int64_t n = c < RG ? k1 - k0 : 0;   // rows past R G (last workgroup) merge nothing

    constexpr int U = unroll<WPR>();
    Merge<E> mg;
    for (int64_t k = part; k < n; k += WPR * U) {
        float l[U];
        float o[U][E];
#pragma unroll
        for (int u = 0; u < U; ++u) {   // past n: row k again, with no weight
            const int64_t kk = k + u * WPR;
            const int64_t row = (k0 + (kk < n ? kk : k)) * RG + c;
            l[u] = kk < n ? p.part_lse[row] : kNegInf;
            const float *src = p.part_o + row * D + lane * E;
#pragma unroll
            for (int e = 0; e < E; ++e) o[u][e] = src[e];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) mg.add(l[u], o[u]);   // skips lse = -inf
    }
    if constexpr (WPR > 1) {
        if (lane == 0) {
            s_m[w] = mg.M;
            s_w[w] = mg.W;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) s_acc[w][lane * E + e] = mg.acc[e];
        __syncthreads();
    }
    if (part != 0 || c >= RG) return;

    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < WPR; ++i) M = fmaxf(M, WPR > 1 ? s_m[w + i] : mg.M);
    // out [B, R, H_q, D]: request b = s / Hkv, KV head h = s % Hkv
    const int64_t out_row =
        ((s / p.Hkv) * p.R + c / G) * (int64_t)(p.Hkv * G) + (s % p.Hkv) * G + c % G;
    __bf16 *out = reinterpret_cast<__bf16 *>(p.out) + out_row * D + lane * E;
    if (M == kNegInf) {   // no live KV: out = 0, lse = -inf
#pragma unroll
        for (int e = 0; e < E; ++e) out[e] = (__bf16)0.f;
        if (p.out_lse && lane == 0) p.out_lse[out_row] = kNegInf;
        return;
    }
    float W = 0.f, acc[E] = {};
    if constexpr (WPR > 1) {
#pragma unroll
        for (int i = 0; i < WPR; ++i) {
            const float cm = s_m[w + i] == kNegInf ? 0.f : __expf(s_m[w + i] - M);
            W += cm * s_w[w + i];
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += cm * s_acc[w + i][lane * E + e];
        }
    } else {
        W = mg.W;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = mg.acc[e];
    }
    const float inv = 1.0f / W;
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = (__bf16)(acc[e] * inv);
    if (p.out_lse && lane == 0) p.out_lse[out_row] = M + __logf(W);
}

template <int D, int WPR>
void launch(const CombineParams &p, hipStream_t stream) {
    constexpr int RPW = kWaves / WPR;
    const int rows = p.R * p.G;
    const dim3 grid((unsigned)p.S, (unsigned)((rows + RPW - 1) / RPW));
    hipLaunchKernelGGL((combine_kernel<D, WPR>), grid, dim3(kThreads), 0, stream, p);
}

}  // namespace

// Waves per row from the mean chunk count of a segment: the dynamic map has
// at most S + P - 1 descriptors over S segments; a static split has `stride`.
hipError_t launch_combine(const CombineParams &p, hipStream_t stream) {
    if (p.S <= 0) return hipSuccess;
    const int64_t chunks = p.seg_off ? (p.S + p.max_chunks - 1) / p.S : p.stride;
    const bool many = chunks >= 8;
    if (p.D == 128) {
        if (many) launch<128, 4>(p, stream); else launch<128, 1>(p, stream);
    } else {
        if (many) launch<64, 4>(p, stream); else launch<64, 1>(p, stream);
    }
    return hipGetLastError();
}

}  // namespace hpcattn
