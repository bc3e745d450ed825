// Persistent paged-KV decode attention (dynamic bins) and the static
// split-KV ablation, sharing one per-tile device path.
//
// "HPC-Ops x SGLang", section "Scheduling around live KV work": at run time
// each persistent workgroup drains its bin; for every descriptor it computes
// attention over one or more contiguous 64-token KV tiles and writes a
// partial output with its log-sum-exp, then moves on until the bin is empty.
// Section "Attention: load balancing for variable-length decode" describes
// the static scheme (fixed grid over KV heads x requests x chunks) that the
// static kernel here reproduces.
//
// Work split on gfx950 (wave64, MFMA):
//   * a workgroup is 4 waves; wave w owns tokens [16 w, 16 w + 16) of every
//     tile, so all 4 waves stay busy even on one-tile descriptors and no
//     barrier is needed inside a descriptor;
//   * one K/V tile (64 tokens of one KV head) serves all G <= 16 query heads
//     of its group: S^T = K Q^T on v_mfma_f32_16x16x32_{bf16,fp8} (16 tokens
//     x 16 head columns, G used), O^T += V^T P^T on v_mfma_f32_16x16x16_bf16;
//   * K and V go straight from HBM to registers with 16-byte loads: lane
//     (r = lane % 16, grp = lane / 16) reads token 16 w + r of K at a d-range
//     that only has to match Q's, and tokens 16 w + 4 grp + j of V at
//     d = r * D/16 .. + D/16, repacked to the MFMA operand with v_perm;
//     these are nontemporal loads, since every KV byte is read once;
//   * the next tile (across descriptor boundaries) is always in flight while
//     the current one is computed;
//   * each wave keeps its own running max / sum / O; the 4 waves are merged
//     in LDS at the end of a descriptor.
// Scores are kept in log2 units (scaled by sm_scale * log2 e) and exp2 is
// the hardware v_exp_f32; the stored LSE is natural-log.
#include "common.h"

namespace hpcattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// Headroom of the softmax reference max, in log2 units: unnormalised weights
// are at most 2^8, far inside bf16 and fp32 range.
constexpr float kSlack = 8.0f;

struct Lane {
    int w, lane, r, grp;
    __device__ Lane() {
        w = threadIdx.x >> 6;
        lane = threadIdx.x & 63;
        r = lane & 15;
        grp = lane >> 4;
    }
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Low (hi = false) or high halves of two dwords: {x.lo16, y.lo16} / {x.hi16, y.hi16}.
template <bool hi>
__device__ __forceinline__ uint32_t halves(uint32_t x, uint32_t y) {
    return __builtin_amdgcn_perm(y, x, hi ? 0x07060302u : 0x05040100u);
}

// Loads at a uniform base plus a 32-bit per-lane byte offset, so that they
// use the scalar-base addressing form (no 64-bit address per lane).
template <class T>
__device__ __forceinline__ T ldg(const void *base, uint32_t off) {
    return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + off);
}

// KV is streamed once per layer: nontemporal loads keep it from displacing
// reusable lines (Q, page ids, the task map) in the caches.
template <class T>
__device__ __forceinline__ T ldg_stream(const void *base, uint32_t off) {
    return __builtin_nontemporal_load(
        reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + off));
}

// Start of the 64-token tile (page, h) of a [num_pages, H_kv, 64, D] pool
// with `esize`-byte elements (uniform across the workgroup).
__device__ __forceinline__ const char *tile_base(const void *pool, int page, int h, int Hkv,
                                                 int row_bytes) {
    return reinterpret_cast<const char *>(pool) +
           ((int64_t)page * Hkv + h) * (int64_t)kTile * row_bytes;
}

// ---------------------------------------------------------------------------
// Element formats.  Each provides the per-lane register image of one tile's
// share of K and V, of the descriptor's Q, and the two MFMA operand builders.
// ---------------------------------------------------------------------------

// bf16 K/V/Q.  QK^T k-step ks covers d = 32 ks + 8 grp + e (e < 8).
template <int D>
struct Bf16 {
    static constexpr int KS = D / 32;   // k-steps of 16x16x32
    static constexpr int VW = D / 32;   // dwords of V per token per lane
    struct Tile {
        u32x4 k[KS];
        uint32_t v[4][VW];
    };
    struct Q {
        u32x4 q[KS];
    };

    static constexpr int kQRowBytes = D * 2;

    // The MFMA B-operand image of Q (head g = r, d-range of k-step ks and
    // lane group grp) from the LDS copy of the group's rows.
    __device__ static void read_q(const uint32_t *sq, int stride, const Lane &ln, Q &q) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            q.q[ks] = *reinterpret_cast<const u32x4 *>(sq + ln.r * stride + 16 * ks + 4 * ln.grp);
    }

    __device__ static void load_tile(const DecodeParams &p, int page, int h, const Lane &ln,
                                     Tile &t) {
        const char *kb = tile_base(p.k, page, h, p.Hkv, D * 2);
        const char *vb = tile_base(p.v, page, h, p.Hkv, D * 2);
        const uint32_t koff = ((16 * ln.w + ln.r) * D + 8 * ln.grp) * 2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) t.k[ks] = ldg_stream<u32x4>(kb, koff + 64 * ks);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t off = ((16 * ln.w + 4 * ln.grp + j) * D + ln.r * (D / 16)) * 2;
            if constexpr (VW == 4) {
                u32x4 x = ldg_stream<u32x4>(vb, off);
                t.v[j][0] = x[0]; t.v[j][1] = x[1]; t.v[j][2] = x[2]; t.v[j][3] = x[3];
            } else {
                u32x2 x = ldg_stream<u32x2>(vb, off);
                t.v[j][0] = x[0]; t.v[j][1] = x[1];
            }
        }
    }

    // Scores S^T[16 w + 4 grp + i][g = r] in log2 units.
    __device__ static f32x4 scores(const DecodeParams &p, const Q &q, const Tile &t,
                                   float qs, int page, int h, const Lane &ln) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, t.k[ks]), __builtin_bit_cast(bf16x8, q.q[ks]), acc,
                0, 0, 0);
        return acc * p.scale_log2;
    }

    static constexpr bool kScaled = false;

    // V^T operand of d-block blk: {V[t_j][r * D/16 + blk], j < 4} as bf16.
    __device__ static void v_dwords(const Tile &t, uint32_t (&vv)[4][VW]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < VW; ++c) vv[j][c] = t.v[j][c];
    }
};

// fp8 e4m3 K/V/Q with fp32 scales per (token, head) ("Fused attention
// prologue": FP8 Q with per-token per-head scales is passed straight to the
// attention kernel).  QK^T k-step ks covers
// d = 64 (ks / 2) + 16 grp + 8 (ks % 2) + e, for K and Q alike.
template <int D>
struct Fp8 {
    static constexpr int KS = D / 32;   // k-steps of 16x16x32 fp8
    static constexpr int NC = D / 64;   // 16-byte chunks of K per lane
    static constexpr int VB = D / 64;   // dwords of V bytes per token per lane
    static constexpr int VW = D / 32;   // dwords of V once widened to bf16
    struct Tile {
        u32x4 k[NC];
        uint32_t v[4][VB];
        f32x4 ks, vs;                   // k/v scales of tokens 16 w + 4 grp + i
    };
    struct Q {
        u32x4 q[NC];
    };

    static constexpr int kQRowBytes = D;

    __device__ static void read_q(const uint32_t *sq, int stride, const Lane &ln, Q &q) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
            q.q[c] = *reinterpret_cast<const u32x4 *>(sq + ln.r * stride + 16 * c + 4 * ln.grp);
    }

    __device__ static void load_tile(const DecodeParams &p, int page, int h, const Lane &ln,
                                     Tile &t) {
        const char *kb = tile_base(p.k, page, h, p.Hkv, D);
        const char *vb = tile_base(p.v, page, h, p.Hkv, D);
        const uint32_t koff = (16 * ln.w + ln.r) * D + 16 * ln.grp;
#pragma unroll
        for (int c = 0; c < NC; ++c) t.k[c] = ldg_stream<u32x4>(kb, koff + 64 * c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t off = (16 * ln.w + 4 * ln.grp + j) * D + ln.r * (D / 16);
            if constexpr (VB == 2) {
                u32x2 x = ldg_stream<u32x2>(vb, off);
                t.v[j][0] = x[0]; t.v[j][1] = x[1];
            } else {
                t.v[j][0] = ldg_stream<uint32_t>(vb, off);
            }
        }
        // Scales of tokens 16 w + 4 grp + i: one 16-byte run per lane group.
        const uint32_t soff = (16 * ln.w + 4 * ln.grp) * 4;
        t.ks = ldg_stream<f32x4>(tile_base(p.k_scale, page, h, p.Hkv, 4), soff);
        t.vs = ldg_stream<f32x4>(tile_base(p.v_scale, page, h, p.Hkv, 4), soff);
    }

    __device__ static f32x4 scores(const DecodeParams &p, const Q &q, const Tile &t,
                                   float qs, int, int, const Lane &) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = ks >> 1, sub = ks & 1;
            const long a = __builtin_bit_cast(long, u32x2{t.k[c][2 * sub], t.k[c][2 * sub + 1]});
            const long b = __builtin_bit_cast(long, u32x2{q.q[c][2 * sub], q.q[c][2 * sub + 1]});
            acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, acc, 0, 0, 0);
        }
        // q_scale of head r, k_scale of token i, and the softmax scale.
        return acc * t.ks * (qs * p.scale_log2);
    }

    static constexpr bool kScaled = true;

    // Widen each token's D/16 fp8 values to bf16 (exact: every e4m3 value is
    // a bf16 value).
    __device__ static void v_dwords(const Tile &t, uint32_t (&vv)[4][VW]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < VB; ++c) {
                const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t.v[j][c], 1.0f, false);
                const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t.v[j][c], 1.0f, true);
                vv[j][2 * c] = __builtin_bit_cast(uint32_t, lo);
                vv[j][2 * c + 1] = __builtin_bit_cast(uint32_t, hi);
            }
    }
};

// ---------------------------------------------------------------------------
// Per-wave online-softmax state and the 4-wave merge.
// ---------------------------------------------------------------------------

template <int D>
struct State {
    static constexpr int NB = D / 16;   // 16-wide d-blocks of O^T
    f32x4 o[NB];   // O[g = r][d = (4 grp + i) * D/16 + blk] for blk, i
    float m, l;    // running max (log2 units) and sum for head g = r

    __device__ void reset() {
#pragma unroll
        for (int b = 0; b < NB; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        m = kNegInf;
        l = 0.f;
    }
};

// One tile's share for this wave: nv = live tokens of the tile (0 .. 64).
template <class KV, int D>
__device__ __forceinline__ void attend_tile(const DecodeParams &p, const uint32_t *sq,
                                            float qs, const typename KV::Tile &t, int nv,
                                            State<D> &st, const Lane &ln) {
    typename KV::Q q;
    KV::read_q(sq, KV::kQRowBytes / 4 + 4, ln, q);
    f32x4 s = KV::scores(p, q, t, qs, 0, 0, ln);
    const int tok0 = 16 * ln.w + 4 * ln.grp;
    if (nv < kTile) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (tok0 + i >= nv) s[i] = kNegInf;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // The reference max st.m moves only when a tile's max exceeds it by more
    // than kSlack (log2 units), so weights stay <= 2^kSlack and O, l are
    // rescaled (a wave-uniform branch) only on those rare tiles.
    if (__any(mx > st.m + kSlack)) {
        const bool moves = mx > st.m + kSlack;
        const float m_new = moves ? mx : st.m;
        // 1 where the reference is kept (also when it stays -inf), 0 from -inf
        const float alpha = moves ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;
        st.l *= alpha;
#pragma unroll
        for (int b = 0; b < D / 16; ++b) st.o[b] = st.o[b] * alpha;
        st.m = m_new;
    }
    const float m_use = st.m == kNegInf ? 0.f : st.m;
    f32x4 pr;
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(s[i] - m_use);
    float ps = (pr[0] + pr[1]) + (pr[2] + pr[3]);
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    st.l += ps;

    if constexpr (KV::kScaled) pr = pr * t.vs;   // fold the per-token V scale into P
    const s16x4 pb = __builtin_bit_cast(
        s16x4, u32x2{pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3])});

    uint32_t vv[4][D / 32];
    KV::v_dwords(t, vv);
    if (nv < kTile) {   // dead slots may hold NaN: zero them, P is already 0
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (tok0 + j >= nv)
#pragma unroll
                for (int c = 0; c < D / 32; ++c) vv[j][c] = 0u;
    }
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
        // d-blocks 2c and 2c + 1: low and high bf16 of dword c of each token.
        const u32x2 lo = {halves<false>(vv[0][c], vv[1][c]), halves<false>(vv[2][c], vv[3][c])};
        const u32x2 hi = {halves<true>(vv[0][c], vv[1][c]), halves<true>(vv[2][c], vv[3][c])};
        st.o[2 * c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(s16x4, lo), pb, st.o[2 * c], 0, 0, 0);
        st.o[2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(s16x4, hi), pb, st.o[2 * c + 1], 0, 0, 0);
    }
}

// LDS scratch for merging the 4 waves of a workgroup.
template <int D, int GR>
struct MergeLds {
    float o[kWaves][GR][D];
    float m[kWaves][GR];
    float l[kWaves][GR];
    // The current descriptor's Q rows (16 rows, rows >= G zero), each padded
    // by 4 dwords so that the per-tile operand reads are bank-conflict free.
    uint32_t q[16 * (D / 2 + 4)];
};

// Copy the G query rows of (b, h) into the LDS Q rows.  All threads.
template <class KV, int D, int GR>
__device__ __forceinline__ void stage_q(const DecodeParams &p, MergeLds<D, GR> &sm, int b,
                                        int h) {
    constexpr int RW = KV::kQRowBytes / 4, QS = RW + 4;
    const uint32_t *src = reinterpret_cast<const uint32_t *>(
        reinterpret_cast<const char *>(p.q) +
        ((int64_t)b * p.Hq + (int64_t)h * p.G) * KV::kQRowBytes);
    for (int i = threadIdx.x; i < p.G * RW; i += kDecodeThreads)
        sm.q[(i / RW) * QS + i % RW] = src[i];
}

// Merge the waves' states and write partial slot `slot`.  All threads.
template <int D, int GR, class Between>
__device__ __forceinline__ void merge_write(const DecodeParams &p, State<D> &st,
                                            MergeLds<D, GR> &sm, int64_t slot, const Lane &ln,
                                            Between between) {
    const int G = p.G;
    if (ln.r < G) {
        if (ln.grp == 0) {
            sm.m[ln.w][ln.r] = st.m;
            sm.l[ln.w][ln.r] = st.l;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float *dst = &sm.o[ln.w][ln.r][(4 * ln.grp + i) * (D / 16)];
#pragma unroll
            for (int b = 0; b < D / 16; b += 4)
                *reinterpret_cast<f32x4 *>(dst + b) =
                    f32x4{st.o[b][i], st.o[b + 1][i], st.o[b + 2][i], st.o[b + 3][i]};
        }
    }
    __syncthreads();
    for (int e = 4 * threadIdx.x; e < G * D; e += 4 * kDecodeThreads) {
        const int g = e / D, d = e % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][g]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float wsum = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float c = __builtin_amdgcn_exp2f(sm.m[w][g] - M);
                wsum += c * sm.l[w][g];
                acc += c * *reinterpret_cast<const f32x4 *>(&sm.o[w][g][d]);
            }
            acc = acc * (1.0f / wsum);
        }
        *reinterpret_cast<f32x4 *>(p.part_o + (slot * G + g) * D + d) = acc;
        if (d == 0)
            p.part_lse[slot * G + g] =
                M == kNegInf ? kNegInf : (M + log2f(wsum)) * kLn2;
    }
    between();   // e.g. stage the next descriptor's Q: no wave reads it now
    __syncthreads();
}

// ---------------------------------------------------------------------------
// The drain loop over a list of descriptors.
// ---------------------------------------------------------------------------

struct Pos {
    int d;          // descriptor index (partial slot for the dynamic kernel)
    int b, h, t, t1, L;
};

// Wave-uniform by construction (same address for every lane): keep it in a
// scalar register so tile bases use the scalar-base load form.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Field-wise select (a whole-struct ?: would be lowered through memory).
__device__ __forceinline__ Pos pick(bool c, const Pos &a, const Pos &b) {
    return Pos{c ? a.d : b.d, c ? a.b : b.b, c ? a.h : b.h,
               c ? a.t : b.t, c ? a.t1 : b.t1, c ? a.L : b.L};
}

// Descriptors of a bin in the task map.
struct MapSource {
    const int32_t *desc;
    const int32_t *lens;
    __device__ __forceinline__ Pos read(int d) const {
        const int32_t *q = desc + 4 * (int64_t)d;
        const int b = uniform(q[0]);
        return Pos{d, b, uniform(q[1]), uniform(q[2]), uniform(q[3]), uniform(lens[b])};
    }
};

// y = the tile after x in drain order; false at the end of the run
// (descriptors x.d + 1 .. d_end - 1 come from src).  y is written once, from
// SSA values, so that the position stays in registers.
__device__ __forceinline__ bool advance(const MapSource &src, int d_end, const Pos &x, Pos &y) {
    const bool same = x.t + 1 < x.t1;
    const bool next = !same && x.d + 1 < d_end;
    Pos n = x;
    n.t = x.t + 1;
    if (next) n = src.read(x.d + 1);
    y = n;
    return same || next;
}

// Page id and live-token count of the tile at x; a tile outside the page
// table or with a page id outside the pool reads page 0 and counts no token.
__device__ __forceinline__ int locate(const DecodeParams &p, const Pos &x, int &nv) {
    nv = min(kTile, x.L - kTile * x.t);
    int page = x.t < p.max_pages ? uniform(p.page_table[(int64_t)x.b * p.max_pages + x.t]) : -1;
    if ((unsigned)page >= (unsigned)p.num_pages) {
        page = 0;
        nv = 0;
    }
    return page;
}

// fp8: the q_scale of head g = r of (x.b, x.h); 1 for bf16.
template <class KV>
__device__ __forceinline__ float q_scale_of(const DecodeParams &p, const Pos &x, const Lane &ln) {
    if constexpr (KV::kScaled) {
        const int g = ln.r < p.G ? ln.r : 0;
        return p.q_scale[(int64_t)x.b * p.Hq + (int64_t)x.h * p.G + g];
    } else {
        return 1.f;
    }
}

// Drains a run of descriptors tile by tile: while tile i is computed, tile
// i + 1 (across descriptor boundaries) is being loaded into the other
// register buffer.  The run starts at `first` and ends with descriptor
// d_end - 1; partials go to slot d (by_desc) or to slot_base.
template <class KV, int D, int GR>
__device__ __forceinline__ void drain(const DecodeParams &p, MergeLds<D, GR> &sm,
                                      const MapSource &src, const Pos &first, int d_end,
                                      int64_t slot_base, bool by_desc) {
    using Tile = typename KV::Tile;
    const Lane ln;
    State<D> st;
    Pos cur = first;
    int nv_cur;

    // Q rows past G stay zero for the whole kernel.
    for (int i = threadIdx.x; i < 16 * (D / 2 + 4); i += kDecodeThreads) sm.q[i] = 0u;
    __syncthreads();
    stage_q<KV, D, GR>(p, sm, cur.b, cur.h);
    float qs = q_scale_of<KV>(p, cur, ln);
    st.reset();
    Tile ta, tb;
    const int pg = locate(p, cur, nv_cur);
    KV::load_tile(p, pg, cur.h, ln, ta);
    __syncthreads();

    // Issue tile i + 1 into `nxt` (after the last tile, a repeat of it that
    // keeps the steady-state path branch-free), compute tile i from `now`,
    // close its descriptor if it ends, staging the next descriptor's Q in
    // LDS inside the merge's barriers.
    auto step = [&](Tile &now, Tile &nxt) __attribute__((always_inline)) -> bool {
        Pos n;
        const bool more = advance(src, d_end, cur, n);
        const Pos far = pick(more, n, cur);
        int nv_n;
        const int pg_n = locate(p, far, nv_n);
        KV::load_tile(p, pg_n, far.h, ln, nxt);

        attend_tile<KV, D>(p, sm.q, qs, now, nv_cur, st, ln);

        if (!more || n.d != cur.d) {
            merge_write<D, GR>(p, st, sm, by_desc ? (int64_t)cur.d : slot_base, ln, [&] {
                if (more) stage_q<KV, D, GR>(p, sm, n.b, n.h);
            });
            if (!more) return false;
            qs = q_scale_of<KV>(p, n, ln);
            st.reset();
        }
        cur = n;
        nv_cur = nv_n;
        return true;
    };
    while (true) {
        if (!step(ta, tb)) break;
        if (!step(tb, ta)) break;
    }
}

// Three workgroups per CU (12 waves) keep enough KV loads in flight; the
// kernel is written to fit the 168 registers per lane that allows.
template <class KV, int D, int GR>
__global__ void __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(3)))
decode_kernel(DecodeParams p) {
    __shared__ MergeLds<D, GR> sm;
    const MapLayout lay(p.B, p.Hkv, p.P);
    const int32_t *bin_off = p.map + lay.bin_off;
    const int d0 = uniform(bin_off[blockIdx.x]), d1 = uniform(bin_off[blockIdx.x + 1]);
    if (d0 >= d1) return;
    const MapSource src{p.map + lay.desc, p.map + lay.lens};
    drain<KV, D, GR>(p, sm, src, src.read(d0), d1, 0, true);
}

template <class KV, int D, int GR>
__global__ void __launch_bounds__(kDecodeThreads)
static_decode_kernel(DecodeParams p) {
    __shared__ MergeLds<D, GR> sm;
    const int64_t slot = blockIdx.x;
    const int64_t seg = slot / p.splits;
    const int k = (int)(slot % p.splits);
    const int b = (int)(seg / p.Hkv), h = (int)(seg % p.Hkv);
    const int L = max(p.seq_lens[b], 0);
    const int64_t n = (L + kTile - 1) / kTile;
    int64_t t0, t1;
    if (p.policy == 0) {
        t0 = k * n / p.splits;
        t1 = (k + 1) * n / p.splits;
    } else {
        const int64_t ct = p.param / kTile;
        t0 = min<int64_t>(n, k * ct);
        t1 = min<int64_t>(n, (k + 1) * ct);
    }
    if (t0 >= t1) {   // an empty split: no weight in the combine
        if (threadIdx.x < p.G) p.part_lse[slot * p.G + threadIdx.x] = kNegInf;
        return;
    }
    // The same drain as the dynamic kernel, over one range and no map: with
    // d_end = 1 and the range numbered 0 it never reads a descriptor.
    drain<KV, D, GR>(p, sm, MapSource{nullptr, nullptr}, Pos{0, b, h, (int)t0, (int)t1, L}, 1,
                     slot, false);
}

template <template <int> class KV, int D>
hipError_t launch_for(const DecodeParams &p, hipStream_t stream, bool dynamic, int grid) {
    if (p.G <= 8) {
        if (dynamic)
            hipLaunchKernelGGL((decode_kernel<KV<D>, D, 8>), dim3(grid), dim3(kDecodeThreads), 0,
                               stream, p);
        else
            hipLaunchKernelGGL((static_decode_kernel<KV<D>, D, 8>), dim3(grid),
                               dim3(kDecodeThreads), 0, stream, p);
    } else {
        if (dynamic)
            hipLaunchKernelGGL((decode_kernel<KV<D>, D, 16>), dim3(grid), dim3(kDecodeThreads),
                               0, stream, p);
        else
            hipLaunchKernelGGL((static_decode_kernel<KV<D>, D, 16>), dim3(grid),
                               dim3(kDecodeThreads), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t dispatch(const DecodeParams &p, int head_dim, int kv_dtype, hipStream_t stream,
                    bool dynamic, int grid) {
    if (grid <= 0) return hipSuccess;
    if (kv_dtype == HPCATTN_KV_BF16)
        return head_dim == 128 ? launch_for<Bf16, 128>(p, stream, dynamic, grid)
                               : launch_for<Bf16, 64>(p, stream, dynamic, grid);
    return head_dim == 128 ? launch_for<Fp8, 128>(p, stream, dynamic, grid)
                           : launch_for<Fp8, 64>(p, stream, dynamic, grid);
}

}  // namespace

int32_t decode_resident_per_cu(int32_t head_dim, int32_t kv_dtype, int32_t group) {
    int n = 0;
    const void *fn;
    const bool small = group <= 8;
    if (kv_dtype == HPCATTN_KV_BF16)
        fn = head_dim == 128 ? (small ? (const void *)decode_kernel<Bf16<128>, 128, 8>
                                      : (const void *)decode_kernel<Bf16<128>, 128, 16>)
                             : (small ? (const void *)decode_kernel<Bf16<64>, 64, 8>
                                      : (const void *)decode_kernel<Bf16<64>, 64, 16>);
    else
        fn = head_dim == 128 ? (small ? (const void *)decode_kernel<Fp8<128>, 128, 8>
                                      : (const void *)decode_kernel<Fp8<128>, 128, 16>)
                             : (small ? (const void *)decode_kernel<Fp8<64>, 64, 8>
                                      : (const void *)decode_kernel<Fp8<64>, 64, 16>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kDecodeThreads, 0) != hipSuccess)
        return 0;
    return n;
}

hipError_t launch_decode(const DecodeParams &p, int32_t head_dim, int32_t kv_dtype,
                         hipStream_t stream) {
    return dispatch(p, head_dim, kv_dtype, stream, true, p.P);
}

hipError_t launch_static_decode(const DecodeParams &p, int32_t head_dim, int32_t kv_dtype,
                                hipStream_t stream) {
    const int64_t grid = (int64_t)p.B * p.Hkv * p.splits;
    return dispatch(p, head_dim, kv_dtype, stream, false, (int)grid);
}

}  // namespace hpcattn
