// The attention prologue after the QKV projection, fused into one kernel.
//
// "HPC-Ops x SGLang", section "Fused attention prologue": QK-Norm before
// RoPE, Q emitted in FP8 with a per-token per-head scale and handed to the
// attention kernel as is, K and V written straight into the paged FP8
// cache.  "Hy3 preview full-stack inference optimization", section 2.2.1:
// RoPE, RMSNorm, an optional Hadamard rotation, quantisation and the KV
// store run as one kernel that keeps every intermediate in registers.
//
// A wave handles four heads of one token; lane l holds elements
// E l .. E l + E - 1 (E = D / 64), so a head row is one coalesced read.  RoPE pairs (i, i+D/2)
// sit in lanes l and l ^ 32; Hadamard stage h pairs lane l with l ^ (h / E)
// (h >= E) or stays in the lane (h < E).  Reductions (sum of squares, amax)
// are wave shuffles.  The RoPE angle pos * base^(-2i/D) is reduced modulo
// 2 pi in fp64 before the fp32 sine and cosine (positions reach 2^17).
#include "common.h"

namespace hpcattn {
namespace {

constexpr int kWavesPerGroup = 4;
constexpr int kHeadsPerWave = 4;
constexpr float kE4M3Max = 448.0f;

// Lane exchanges.  xor masks below 32 use ds_swizzle in its bit mode (the
// pattern lane ^ m is encoded in the instruction, no address operand);
// the xor-32 exchange uses ds_bpermute with an address computed once.
template <int M>
__device__ __forceinline__ float xor_lanes(float v) {
    static_assert(M >= 1 && M < 32, "swizzle masks stay within 32 lanes");
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (M << 10)));
}

__device__ __forceinline__ float xor32(float v, int addr32) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(addr32, __float_as_int(v)));
}

// Sum / max over all 64 lanes: within each half by swizzles, then the two
// halves' lane-0 values (the result is wave-uniform).
__device__ __forceinline__ float wave_sum(float v) {
    v += xor_lanes<1>(v);
    v += xor_lanes<2>(v);
    v += xor_lanes<4>(v);
    v += xor_lanes<8>(v);
    v += xor_lanes<16>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, xor_lanes<1>(v));
    v = fmaxf(v, xor_lanes<2>(v));
    v = fmaxf(v, xor_lanes<4>(v));
    v = fmaxf(v, xor_lanes<8>(v));
    v = fmaxf(v, xor_lanes<16>(v));
    return fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)));
}

// One cross-lane Hadamard stage with partner lane l ^ LM: the lane with the
// LM bit clear keeps a + b, the other b - a, i.e. partner + sign * self.
template <int LM>
__device__ __forceinline__ float butterfly(float v, int lane, int addr32) {
    const float o = LM == 32 ? xor32(v, addr32) : xor_lanes<(LM < 32 ? LM : 1)>(v);
    const float sgn = (lane & LM) ? -1.f : 1.f;
    return fmaf(sgn, v, o);
}

// Workgroup (t, head block y): token t; wave w takes `chunks` groups of four
// heads, group c covering heads 4 (w + 4 (c + chunks y)) ..  Everything that
// depends only on the token and the lane -- the RoPE angles' sines and
// cosines, the norm weights -- is computed once per wave and reused for all
// its heads (chunks > 1 for large token counts: one workgroup per token).
template <int D>
__global__ void __launch_bounds__(64 * kWavesPerGroup) prologue_kernel(PrologueParams p) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x;
    const int heads = p.Hq + 2 * p.Hkv;
    const int w = threadIdx.x >> 6;
    const int first = (blockIdx.y * p.chunks * kWavesPerGroup + w) * kHeadsPerWave;
    if (first >= heads) return;   // whole waves only
    const __bf16 *src = reinterpret_cast<const __bf16 *>(p.qkv) + ((int64_t)t * heads) * D + E * lane;

    // RoPE sines and cosines of this lane's elements at position p.positions[t]:
    // theta_i = pos * base^(-2i/D), reduced modulo 2 pi in fp64.
    float sn[E], cs[E];
    const bool rope = (p.flags & HPCATTN_PROLOGUE_ROPE) && first < p.Hq + p.Hkv;
    if (rope) {
        const double pos = (double)p.positions[t];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = E * (lane & 31) + e;   // pair index < D/2
            const double ang = pos * exp2(-(2.0 * i / D) * p.log2_base);
            const double red = ang - 6.283185307179586 * floor(ang * 0.15915494309189535);
            sincosf((float)red, &sn[e], &cs[e]);
            if (lane < 32) sn[e] = -sn[e];   // lower half: x_i c - x_{i+D/2} s
        }
    }
    float wq[E], wk[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        wq[e] = p.q_norm_w ? p.q_norm_w[E * lane + e] : 1.f;
        wk[e] = p.k_norm_w ? p.k_norm_w[E * lane + e] : 1.f;
    }
    const int addr32 = (lane ^ 32) << 2;   // ds_bpermute byte address of lane l ^ 32
    const int slot = p.cache_slots[t];
    const bool store_kv = slot >= 0 && (slot >> 6) < p.num_pages;

    for (int c = 0; c < p.chunks; ++c) {
    const int j0 = first + c * kWavesPerGroup * kHeadsPerWave;
    if (j0 >= heads) break;
    const int j1 = min(heads, j0 + kHeadsPerWave);

    // Rows of this chunk's heads, loaded together.
    float x[kHeadsPerWave][E];
#pragma unroll
    for (int u = 0; u < kHeadsPerWave; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e) x[u][e] = (float)src[min(j0 + u, j1 - 1) * D + e];   // in-row

#pragma unroll
    for (int u = 0; u < kHeadsPerWave; ++u) {
        const int j = j0 + u;
        if (j >= j1) break;
        const int kind = j < p.Hq ? 0 : (j < p.Hq + p.Hkv ? 1 : 2);   // Q, K, V (uniform)
        const int hh = kind == 0 ? j : (kind == 1 ? j - p.Hq : j - p.Hq - p.Hkv);
        if (kind != 0 && !store_kv) continue;
        float *v = x[u];
        if (kind < 2) {
            if (kind == 0 ? p.q_norm_w != nullptr : p.k_norm_w != nullptr) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) ss += v[e] * v[e];
                const float inv = rsqrtf(wave_sum(ss) / D + p.eps);
#pragma unroll
                for (int e = 0; e < E; ++e) v[e] = v[e] * inv * (kind == 0 ? wq[e] : wk[e]);
            }
            if (rope) {   // (x_i, x_{i+D/2}) in lanes l, l ^ 32; sn carries the sign
#pragma unroll
                for (int e = 0; e < E; ++e) v[e] = fmaf(xor32(v[e], addr32), sn[e], v[e] * cs[e]);
            }
            if (p.flags & HPCATTN_PROLOGUE_HADAMARD) {   // y = H_D x / sqrt(D)
#pragma unroll
                for (int h = 1; h < E; h <<= 1)
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        if (e & h) continue;
                        const float a = v[e], b = v[e | h];
                        v[e] = a + b;
                        v[e | h] = a - b;
                    }
#pragma unroll
                for (int e = 0; e < E; ++e) {   // stages h = E .. D/2: partner lane l ^ (h / E)
                    v[e] = butterfly<1>(v[e], lane, addr32);
                    v[e] = butterfly<2>(v[e], lane, addr32);
                    v[e] = butterfly<4>(v[e], lane, addr32);
                    v[e] = butterfly<8>(v[e], lane, addr32);
                    v[e] = butterfly<16>(v[e], lane, addr32);
                    v[e] = butterfly<32>(v[e], lane, addr32);
                }
                const float norm = rsqrtf((float)D);
#pragma unroll
                for (int e = 0; e < E; ++e) v[e] *= norm;
            }
        }

        // Destination row: the Q output, or the token's cache slot.
        const int64_t row = kind == 0 ? (int64_t)t * p.Hq + hh
                                      : ((int64_t)(slot >> 6) * p.Hkv + hh) * kTile +
                                            (slot & (kTile - 1));
        void *dst = kind == 0 ? p.q_out : (kind == 1 ? p.k_pages : p.v_pages);
        if (p.kv_dtype == HPCATTN_KV_BF16) {
            __bf16 *o = reinterpret_cast<__bf16 *>(dst) + row * D + E * lane;
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = (__bf16)v[e];
            continue;
        }
        // fp8: scale = amax / 448 (1 for an all-zero row), codes = RNE(x / scale).
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
        amax = wave_max(amax);
        const float scale = amax > 0.f ? amax * (1.0f / kE4M3Max) : 1.0f;
        const float rcp = amax > 0.f ? __builtin_amdgcn_rcpf(scale) : 1.0f;
        uint8_t *o = reinterpret_cast<uint8_t *>(dst) + row * D + E * lane;
        float y[E];
#pragma unroll
        for (int e = 0; e < E; ++e) y[e] = fminf(fmaxf(v[e] * rcp, -kE4M3Max), kE4M3Max);
        if constexpr (E == 1) {
            o[0] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y[0], 0.f, 0, false) & 0xFF);
        } else {
            const uint32_t packed = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            *reinterpret_cast<uint16_t *>(o) = (uint16_t)(packed & 0xFFFF);
        }
        if (lane == 0) {
            float *sc = kind == 0 ? p.q_scale : (kind == 1 ? p.k_scale : p.v_scale);
            sc[row] = scale;
        }
    }
    }
}

}  // namespace

hipError_t launch_prologue(const PrologueParams &p, int32_t head_dim, hipStream_t stream) {
    const int heads = p.Hq + 2 * p.Hkv;
    if (p.T <= 0 || heads <= 0) return hipSuccess;
    // Large token counts: one workgroup per token (trig set-up paid once per
    // wave); small ones: 16 heads per workgroup for parallelism.
    const int per_group = kWavesPerGroup * kHeadsPerWave;
    const int blocks = (heads + per_group - 1) / per_group;
    PrologueParams q = p;
    q.chunks = p.T >= 1024 ? blocks : 1;
    const dim3 grid((unsigned)p.T, (unsigned)((blocks + q.chunks - 1) / q.chunks));
    if (head_dim == 128)
        hipLaunchKernelGGL(prologue_kernel<128>, grid, dim3(64 * kWavesPerGroup), 0, stream, q);
    else
        hipLaunchKernelGGL(prologue_kernel<64>, grid, dim3(64 * kWavesPerGroup), 0, stream, q);
    return hipGetLastError();
}

}  // namespace hpcattn
