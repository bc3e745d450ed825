// The attention prologue after the QKV projection, fused into one kernel.
//
// "HPC-Ops x SGLang", section "Fused attention prologue": QK-Norm before
// RoPE, Q emitted in FP8 with a per-token per-head scale and handed to the
// attention kernel as is, K and V written straight into the paged FP8
// cache.  "Hy3 preview full-stack inference optimization", section 2.2.1:
// RoPE, RMSNorm, an optional Hadamard rotation, quantisation and the KV
// store run as one kernel that keeps every intermediate in registers.
//
// The kernel does much VALU work per byte (a wave64 VALU instruction takes
// 4 cycles of its SIMD), so the layout is chosen for the fewest instructions
// per head row; it runs between that issue bound and a read-write HBM
// stream:
//   * a head row sits on the 4 lanes of a quad, 16 rows per wave.  Lane q of
//     the quad holds the D / 4 elements j = 32 m + 8 q + e (e < 8, m < D/32)
//     as 16-byte chunks m, so the quad reads and writes contiguous bytes;
//   * the RoPE partner of element j < D/2 (j + D/2) is in the same lane, and
//     so are 5 (D = 128) or 4 (D = 64) of the Hadamard rotation's butterfly
//     stages; only the 2 stages over q cross lanes;
//   * with both RoPE and the Hadamard rotation, the rotation of the pair
//     (a, b) by angle t and the butterfly stage that pairs the same two
//     elements are one step with coefficients P = cos t + sin t and
//     M = cos t - sin t: (a, b) -> (a P + b M, a M - b P);
//   * a cross-lane stage is one DPP multiply-add per element: the lane's
//     values enter the two stages multiplied by c = s1 s2, s_i = -1 where
//     bit i of q is set (folded into the RoPE coefficients), and then each
//     stage is u <- u + k u', u' the partner lane's value, k = -s_i; the
//     factor is 1 again after the second stage;
//   * the RMS factor 1/sqrt(mean x^2 + eps) and the 1/sqrt(D) of the
//     rotation are per-row scalars applied after the linear steps: folded
//     into the fp8 scale (the codes do not depend on them) or into one
//     multiply of the bf16 output;
//   * the sum of squares reads the bf16 pairs directly (v_dot2_f32_bf16).
// A workgroup takes one token and one wave per 16 heads (measured: more
// tokens per workgroup, which would share the set-up, run slower).  The
// token's RoPE coefficients are computed once and shared through LDS: the
// angle pos * f_i (f_i = base^(-2i/D), computed in fp64 on the host) is
// reduced in fp64 to r + k pi/2 with |r| <= pi/4 (positions reach 2^17), and
// sin r, cos r are Taylor polynomials in fp32 (truncation below 2e-9).
#include "common.h"

namespace hpcattn {
namespace {

constexpr int kRows = 16;        // head rows per wave (a quad each)
constexpr int kMaxWaves = 16;    // waves per workgroup at most (256 heads)
constexpr float kE4M3Max = 448.0f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Lane ^ M within the quad (DPP quad_perm; every lane's source is valid).
template <int M>
__device__ __forceinline__ float xq(float x) {
    static_assert(M == 1 || M == 2, "exchanges within a quad");
    constexpr int kCtrl = M == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2], [2,3,0,1]
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, true));
}

// u[e] += k * (u[e] of lane q ^ M), eight elements, as v_fmac_f32 with a
// DPP source (the compiler does not fold a DPP move into a multiply-add).
// The leading s_nop covers the two wait states a DPP read needs after a
// VALU write of its source; each instruction reads a register no earlier
// one in the block writes.
template <int M>
__device__ __forceinline__ void cross8(float *u, float k) {
    if constexpr (M == 1) {
        asm volatile(
            "s_nop 1\n\t"
            "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
            : "+v"(u[0]), "+v"(u[1]), "+v"(u[2]), "+v"(u[3]), "+v"(u[4]), "+v"(u[5]),
              "+v"(u[6]), "+v"(u[7])
            : "v"(k));
    } else {
        static_assert(M == 2, "exchanges within a quad");
        asm volatile(
            "s_nop 1\n\t"
            "v_fmac_f32_dpp %0, %0, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %1, %1, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %2, %2, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %3, %3, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %4, %4, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %5, %5, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %6, %6, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %7, %7, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
            : "+v"(u[0]), "+v"(u[1]), "+v"(u[2]), "+v"(u[3]), "+v"(u[4]), "+v"(u[5]),
              "+v"(u[6]), "+v"(u[7])
            : "v"(k));
    }
}

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// sin and cos of an angle given in fp64 (|angle| < 2^31): reduced in fp64
// to r + k pi/2, |r| <= pi/4, then Taylor polynomials through r^9 and r^10.
// The reduction's error is k times that of pi/2 in fp64 (6e-17): below 1e-11
// for positions up to 2^17, and about one fp32 ulp of r at |angle| = 2^31.
__device__ __forceinline__ void sincos_reduced(double angle, float &s, float &c) {
    const double kq = rint(angle * 0.6366197723675814);          // 2 / pi
    const float r = (float)fma(-kq, 1.5707963267948966, angle);   // pi / 2
    const float r2 = r * r;
    const float ps = fmaf(fmaf(fmaf(fmaf(r2, 2.7557319e-6f, -1.9841270e-4f), r2, 8.3333333e-3f),
                               r2, -1.6666667e-1f), r2 * r, r);
    const float pc = fmaf(fmaf(fmaf(fmaf(fmaf(r2, -2.7557319e-7f, 2.4801587e-5f), r2,
                                         -1.3888889e-3f), r2, 4.1666667e-2f), r2, -0.5f),
                          r2, 1.0f);
    const int k = (int)(int64_t)kq & 3;   // sin(r + k pi/2), cos(r + k pi/2)
    const float a = (k & 1) ? pc : ps, b = (k & 1) ? ps : pc;
    s = (k & 2) ? -a : a;
    c = ((k + 1) & 2) ? -b : b;
}

template <int D>
struct Lay {
    static constexpr int E = D / 4;        // elements per lane
    static constexpr int NCH = D / 32;     // 8-element chunks per lane
    static constexpr int HCH = NCH / 2;    // chunks of the lower half
    static constexpr int TOP = 8 * HCH;    // lane index bit of element bit D/2
};

// Workgroup (x, y): token x; wave w the chunk of heads 16 c .. 16 c + 15,
// c = waves y + w.
template <int D, bool ROPE, bool HAD, bool FP8>
__global__ void __launch_bounds__(64 * kMaxWaves) prologue_kernel(PrologueParams p) {
    using L = Lay<D>;
    constexpr int E = L::E;
    constexpr int NCH = L::NCH;
    constexpr int HALF = D / 2;
    // RoPE coefficients of the token: [sign c][A or B][angle index]
    __shared__ float trig[2][2][HALF];
    __shared__ float wts[2][D];   // q_norm_w, k_norm_w
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int waves = blockDim.x >> 6;
    const int r = lane >> 2;   // row of the wave
    const int q = lane & 3;    // lane within the row
    const int heads = p.Hq + 2 * p.Hkv;
    const int64_t t = blockIdx.x;

    // Set-up shared by the workgroup: norm weights, and the RoPE coefficients
    // (A, B) = (P, M) with the Hadamard rotation, else (cos, sin); the second
    // sign holds -A, -B for lanes whose values carry c = -1.
    for (int i = threadIdx.x; i < 2 * D; i += blockDim.x) {
        const float *src = i < D ? p.q_norm_w : p.k_norm_w;
        wts[i / D][i % D] = src ? src[i % D] : 1.f;
    }
    if constexpr (ROPE) {
        for (int a = threadIdx.x; a < HALF; a += blockDim.x) {
            float sv, cv;
            sincos_reduced((double)p.positions[t] * p.freq[a], sv, cv);
            const float A = HAD ? cv + sv : cv, B = HAD ? cv - sv : sv;
            trig[0][0][a] = A;
            trig[0][1][a] = B;
            trig[1][0][a] = -A;
            trig[1][1][a] = -B;
        }
    }
    __syncthreads();

    const int j = kRows * (blockIdx.y * waves + w) + r;   // this lane's head
    if (kRows * (blockIdx.y * waves + w) >= heads) return;   // whole waves only
    const bool valid = j < heads;
    const int kind = j < p.Hq ? 0 : (j < p.Hq + p.Hkv ? 1 : 2);   // Q, K, V (dead rows: V)
    const int hh = kind == 0 ? j : (kind == 1 ? j - p.Hq : j - p.Hq - p.Hkv);
    const bool norm = kind == 0 ? p.q_norm_w != nullptr : (kind == 1 && p.k_norm_w != nullptr);
    const float *wrow = wts[kind == 0 ? 0 : 1];
    const int csgn = (q == 1 || q == 2) ? 1 : 0;   // c = s1 s2 = -1
    const float k1 = (q & 1) ? 1.f : -1.f;         // -s1
    const float k2 = (q & 2) ? 1.f : -1.f;         // -s2

    // The row's D / 4 bf16 elements of token t, as 16-byte chunks (a dead
    // row reads a valid row and stores nothing).
    const uint16_t *qkv = reinterpret_cast<const uint16_t *>(p.qkv);
    const int src_head = valid ? j : heads - 1;
    uint4 x[NCH];
    const uint16_t *src = qkv + (t * heads + src_head) * D + 8 * q;
#pragma unroll
    for (int m = 0; m < NCH; ++m) x[m] = *reinterpret_cast<const uint4 *>(src + 32 * m);
    const uint32_t *xw = reinterpret_cast<const uint32_t *>(x);   // bf16 pairs
    float v[E];
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
        v[2 * i] = __uint_as_float(xw[i] << 16);
        v[2 * i + 1] = __uint_as_float(xw[i] & 0xFFFF0000u);
    }
    float f = 1.f;   // the row's scalar factor, applied at the end
    if (kind < 2) {   // Q or K: QK-Norm, RoPE, Hadamard (lanes of V rows skip)
        if (norm) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < E / 2; ++i) {
                const bf16x2 b2 = __builtin_bit_cast(bf16x2, xw[i]);
                ss = __builtin_amdgcn_fdot2_f32_bf16(b2, b2, ss, false);
            }
            ss += xq<1>(ss);
            ss += xq<2>(ss);
            f = rsqrtf(ss * (1.0f / D) + p.eps);
#pragma unroll
            for (int m = 0; m < NCH; ++m)   // element j = 32 m + 8 q + e at index 8 m + e
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float4 wv =
                        *reinterpret_cast<const float4 *>(wrow + 32 * m + 8 * q + 4 * h);
                    float *c = v + 8 * m + 4 * h;
                    c[0] *= wv.x;
                    c[1] *= wv.y;
                    c[2] *= wv.z;
                    c[3] *= wv.w;
                }
        }
        if constexpr (ROPE) {   // element index k pairs with k + TOP
            const float *ta = trig[HAD ? csgn : 0][0];
            const float *tb = trig[HAD ? csgn : 0][1];
#pragma unroll
            for (int m = 0; m < L::HCH; ++m)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i = 32 * m + 8 * q + 4 * h;   // angle index of element 8 m + 4 h
                    const float4 a4 = *reinterpret_cast<const float4 *>(ta + i);
                    const float4 b4 = *reinterpret_cast<const float4 *>(tb + i);
                    const float ca[4] = {a4.x, a4.y, a4.z, a4.w};
                    const float cb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int k = 8 * m + 4 * h + e;
                        const float a = v[k], b = v[k + L::TOP];
                        if constexpr (HAD) {   // rotation and the butterfly over bit D/2
                            v[k] = fmaf(a, ca[e], b * cb[e]);
                            v[k + L::TOP] = fmaf(a, cb[e], -(b * ca[e]));
                        } else {
                            v[k] = fmaf(a, ca[e], -(b * cb[e]));
                            v[k + L::TOP] = fmaf(b, ca[e], a * cb[e]);
                        }
                    }
                }
        }
        if constexpr (HAD) {   // y = H_D x / sqrt(D): in-lane stages, then the two over q
            if constexpr (!ROPE) {   // the factor c the cross-lane stages expect
                const float c = csgn ? -1.f : 1.f;
#pragma unroll
                for (int e = 0; e < E; ++e) v[e] *= c;
            }
#pragma unroll
            for (int hb = 1; hb < E; hb <<= 1) {
                if (ROPE && hb == L::TOP) continue;   // done with the rotation
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    if (k & hb) continue;
                    const float a = v[k], b = v[k | hb];
                    v[k] = a + b;
                    v[k | hb] = a - b;
                }
            }
#pragma unroll
            for (int e = 0; e < E; e += 8) cross8<1>(v + e, k1);
#pragma unroll
            for (int e = 0; e < E; e += 8) cross8<2>(v + e, k2);
            f *= D == 128 ? 0.08838834764831845f : 0.125f;   // 1/sqrt(D)
        }
    }

    // Destination row: the Q output, or the token's cache slot.
    const int slot = p.cache_slots[t];
    const bool store = valid && (kind == 0 || (slot >= 0 && (slot >> 6) < p.num_pages));
    const int64_t row = kind == 0 ? t * p.Hq + hh
                                  : ((int64_t)(slot >> 6) * p.Hkv + hh) * kTile +
                                        (slot & (kTile - 1));
    void *dst = kind == 0 ? p.q_out : (kind == 1 ? p.k_pages : p.v_pages);
    if constexpr (!FP8) {
        if (store) {
            uint16_t *out = reinterpret_cast<uint16_t *>(dst) + row * D + 8 * q;
#pragma unroll
            for (int m = 0; m < NCH; ++m) {
                const float *c = v + 8 * m;
                *reinterpret_cast<uint4 *>(out + 32 * m) =
                    uint4{pack2_bf16(c[0] * f, c[1] * f), pack2_bf16(c[2] * f, c[3] * f),
                          pack2_bf16(c[4] * f, c[5] * f), pack2_bf16(c[6] * f, c[7] * f)};
            }
        }
        return;
    }
    // fp8: scale = amax(f v) / 448 (1 for an all-zero row), codes =
    // RNE(f v / scale) = RNE(v * 448 / amax(v)).  |v * rcp| stays below
    // 448 (1 + 2^-22) (rcp is within 1 ulp), which rounds to 448, so the
    // conversion never sees a value beyond the format's range.
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
    amax = fmaxf(amax, xq<1>(amax));
    amax = fmaxf(amax, xq<2>(amax));
    const float amax_y = amax * f;
    const bool nz = amax_y > 0.f;
    const float scale = nz ? amax_y * (1.0f / kE4M3Max) : 1.0f;
    const float rcp = nz ? kE4M3Max * __builtin_amdgcn_rcpf(amax) : 0.0f;
    if (store) {
        uint8_t *out = reinterpret_cast<uint8_t *>(dst) + row * D + 8 * q;
#pragma unroll
        for (int m = 0; m < NCH; ++m) {
            uint32_t o[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float *c = v + 8 * m + 4 * h;
                int packed = __builtin_amdgcn_cvt_pk_fp8_f32(c[0] * rcp, c[1] * rcp, 0, false);
                packed = __builtin_amdgcn_cvt_pk_fp8_f32(c[2] * rcp, c[3] * rcp, packed, true);
                o[h] = (uint32_t)packed;
            }
            *reinterpret_cast<uint2 *>(out + 32 * m) = uint2{o[0], o[1]};
        }
        if (q == 0) {
            float *sc = kind == 0 ? p.q_scale : (kind == 1 ? p.k_scale : p.v_scale);
            sc[row] = scale;
        }
    }
}

}  // namespace

hipError_t launch_prologue(const PrologueParams &p, int32_t head_dim, hipStream_t stream) {
    const int heads = p.Hq + 2 * p.Hkv;
    if (p.T <= 0 || heads <= 0) return hipSuccess;
    // One workgroup per token, one wave per 16 heads (at most 16 waves per
    // workgroup, more workgroups along y beyond 256 heads).
    const int64_t chunks = (heads + kRows - 1) / kRows;
    const int waves = (int)std::min<int64_t>(chunks, kMaxWaves);
    const dim3 grid((unsigned)p.T, (unsigned)((chunks + waves - 1) / waves));
    using Kernel = void (*)(PrologueParams);
    // [head_dim == 128][ROPE][HADAMARD][fp8]
    static constexpr Kernel kKernels[2][2][2][2] = {
        {{{prologue_kernel<64, false, false, false>, prologue_kernel<64, false, false, true>},
          {prologue_kernel<64, false, true, false>, prologue_kernel<64, false, true, true>}},
         {{prologue_kernel<64, true, false, false>, prologue_kernel<64, true, false, true>},
          {prologue_kernel<64, true, true, false>, prologue_kernel<64, true, true, true>}}},
        {{{prologue_kernel<128, false, false, false>, prologue_kernel<128, false, false, true>},
          {prologue_kernel<128, false, true, false>, prologue_kernel<128, false, true, true>}},
         {{prologue_kernel<128, true, false, false>, prologue_kernel<128, true, false, true>},
          {prologue_kernel<128, true, true, false>, prologue_kernel<128, true, true, true>}}}};
    const Kernel k = kKernels[head_dim == 128][(p.flags & HPCATTN_PROLOGUE_ROPE) != 0]
                             [(p.flags & HPCATTN_PROLOGUE_HADAMARD) != 0]
                             [p.kv_dtype == HPCATTN_KV_FP8_E4M3];
    hipLaunchKernelGGL(k, grid, dim3(64 * waves), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hpcattn
