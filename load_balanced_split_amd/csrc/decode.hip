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
// Two device paths.  The per-wave path (up to 16 query rows per KV head:
// plain decode, G <= 16) is described here; the shared-tile path for more
// rows (multi-row draft verification) is described at its own section.
//
// Work split on gfx950 (wave64, MFMA), per-wave path:
//   * a workgroup is 4 waves; wave w owns tokens [16 w, 16 w + 16) of every
//     tile, so all 4 waves stay busy even on one-tile descriptors and no
//     barrier is needed inside a descriptor;
//   * one K/V tile (64 tokens of one KV head) serves every query row of its
//     group (G heads, times R rows of a multi-row step, R G <= 16) as 16 MFMA
//     columns: S^T = K Q^T on v_mfma_f32_16x16x32_{bf16,fp8} (16 tokens x 16
//     columns), O^T += V^T P^T on v_mfma_f32_16x16x16_bf16;
//   * K and V go from HBM to registers with 16-byte loads: lane
//     (r = lane % 16, grp = lane / 16) holds token 16 w + r of K at a
//     d-range that only has to match Q's (bf16: loaded in that shape; fp8:
//     loaded in whole rows and reordered through the wave's LDS rows, see
//     "K rows through LDS"), and tokens 16 w + 4 grp + j of V at
//     d = r * D/16 .. + D/16, repacked to the MFMA operand with v_perm;
//     these are nontemporal buffer loads (every KV byte is read once)
//     bounded at the tile's live rows, so dead rows read as zero and cost
//     no memory traffic;
//   * the next tile (across descriptor boundaries) is always in flight while
//     the current one is computed; page ids and descriptors are read through
//     the scalar memory path (their waits do not count the KV loads), the
//     next descriptor as soon as the current one is entered;
//   * each wave keeps its own running max / O and, per lane, the sum of its
//     own tokens' weights; the column reductions across lanes happen only
//     when the reference max moves and at the end of a descriptor, where
//     the 4 waves are merged in LDS.
// Scores are kept in log2 units (scaled by sm_scale * log2 e) and exp2 is
// the hardware v_exp_f32; the stored LSE is natural-log.
#include <atomic>

#include "common.h"

namespace hpcattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
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

// Query rows per request: MR (multi-row) kernels read R from the arguments,
// the others are compiled for R = 1.
template <bool MR>
__device__ __forceinline__ int rows_per_req(const DecodeParams &p) {
    return MR ? p.R : 1;
}

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

// Start of the 64-token tile (page, h) of a [num_pages, H_kv, 64, D] pool
// with `esize`-byte elements (uniform across the workgroup).
__device__ __forceinline__ const char *tile_base(const void *pool, int page, int h, int Hkv,
                                                 int row_bytes) {
    return reinterpret_cast<const char *>(pool) +
           ((int64_t)page * Hkv + h) * (int64_t)kTile * row_bytes;
}

// Raw buffer resources (stride 0, word 3 of a plain untyped buffer).  A
// dword of a buffer load at or past num_records bytes reads 0 without a
// memory access, and a store there writes nothing.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kNontemporal = 2;   // cache policy nt: streamed once

// `base` and `bytes` must be wave-uniform: they are read from the first
// active lane, so that the resource lives in scalar registers (a resource
// the compiler takes for divergent is used through a loop over its values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void *base, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo),
                                             (short)0, __builtin_amdgcn_readfirstlane(bytes),
                                             kRawBufferWord3);
}

// The live rows of tile (page, h): tokens [0, live) of its 64, where `nv`
// is the request's tokens from the tile's first on (clamped here).  Dead
// rows read as zero and cost no HBM traffic; live = 0 reads nothing at all.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t live_rows(const void *pool, int page, int h,
                                                             int Hkv, int row_bytes, int nv) {
    const int live = min(max(nv, 0), kTile);
    return span_rsrc(tile_base(pool, page, h, Hkv, row_bytes), live * row_bytes);
}

// A lane's byte offset, opaque to the optimiser at the point of use, so
// that offset + constant folds into the load's immediate offset instead of
// each sum being hoisted out of the loop into a register of its own.
__device__ __forceinline__ uint32_t lane_off(uint32_t off) {
    asm volatile("" : "+v"(off));
    return off;
}

// Nontemporal buffer loads of 4, 2 or 1 dwords at a byte offset.  KV is
// streamed once per layer: nontemporal loads keep it from displacing
// reusable lines (Q, page ids, the task map) in the caches.
__device__ __forceinline__ u32x4 ldb4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNontemporal);
}
__device__ __forceinline__ u32x2 ldb2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kNontemporal);
}
__device__ __forceinline__ uint32_t ldb1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kNontemporal);
}

// A 16-byte buffer load with the default (temporal) cache policy, for lines
// that a second wave reads soon after the first.
__device__ __forceinline__ u32x4 ldb4_keep(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Wave-uniform by construction (same address for every lane): keep it in a
// scalar register so tile bases use the scalar-base load form.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// A read-only int32 at a wave-uniform index, through the scalar memory path
// (constant address space): its wait counts scalar loads only, so it never
// waits for the KV tiles in flight on the vector memory path.
__device__ __forceinline__ int sload(const int32_t *base, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t *)base)[i];
}

// ---------------------------------------------------------------------------
// K rows through LDS.  The QK^T operand wants token r of a 16-token block in
// lane r + 16 grp, 16 bytes of it per lane (MFMA rows are lanes mod 16).
// Loaded in that shape straight from HBM, every load instruction takes one
// 64-byte piece of each of 16 token rows, and such loads stream about 15%
// (256-byte bf16 rows) to 20% (128-byte fp8 rows) slower than loads of
// whole rows.  So fp8 K is loaded in whole rows (load c, lane l: bytes
// 1024 c + 16 l of the wave's 16 rows) and each wave passes it through 16
// rows of its own LDS, padded to CPR + 1 chunks of 16 bytes (CPR chunks per
// row): the 16 lanes of a quarter-wave reading one chunk of 16 rows hit 16
// distinct bank groups, and every address is a per-lane base plus a
// constant.  The same wave stores and reads, and a wave's LDS operations run
// in order, so no barrier is needed.  bf16 K keeps the operand-shaped loads:
// on its wider rows the loss is smaller than the cost of the round trip.
// ---------------------------------------------------------------------------

// Bytes of a wave's padded K rows.
template <int CPR>
constexpr int k_rows_bytes() {
    return 16 * (CPR + 1) * 16;
}

// In: k[c] = bytes 1024 c + 16 lane of the wave's rows.  Out: k[c] = chunk
// 4 c + grp of token r (the operand of k-step c, or of k-steps 2c, 2c+1 for
// fp8).
template <int CPR>
__device__ __forceinline__ void k_to_operand(uint8_t *rows, int lane, int r, int grp,
                                             u32x4 (&k)[CPR / 4]) {
    constexpr int S = CPR + 1;   // padded row stride in chunks
    uint8_t *wr = rows + 16 * (S * (lane / CPR) + lane % CPR);
#pragma unroll
    for (int c = 0; c < CPR / 4; ++c)
        *reinterpret_cast<u32x4 *>(wr + 16 * S * (64 / CPR) * c) = k[c];
    // other lanes' stores above, this lane's loads below: keep the order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint8_t *rd = rows + 16 * (S * r + grp);
#pragma unroll
    for (int c = 0; c < CPR / 4; ++c) k[c] = *reinterpret_cast<const u32x4 *>(rd + 64 * c);
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

    // K is loaded in the operand shape: no LDS rows.
    static constexpr bool kKRows = false;
    __device__ static void k_operand(uint8_t *, const Lane &, Tile &) {}

    // The MFMA B-operand image of Q (head g = r, d-range of k-step ks and
    // lane group grp) from the LDS copy of the group's rows.
    __device__ static void read_q(const uint32_t *sq, int stride, const Lane &ln, Q &q) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            q.q[ks] = *reinterpret_cast<const u32x4 *>(sq + ln.r * stride + 16 * ks + 4 * ln.grp);
    }

    // The wave's share of tile (page, h) with nv tokens from its first on:
    // dead rows (token >= nv) read as zero.
    __device__ static void load_tile(const DecodeParams &p, int page, int h, int nv,
                                     const Lane &ln, Tile &t) {
        const auto kr = live_rows(p.k, page, h, p.Hkv, D * 2, nv);
        const auto vr = live_rows(p.v, page, h, p.Hkv, D * 2, nv);
        // K straight in the operand shape: the 256-byte rows lose less to
        // the piecewise row reads than the LDS round trip costs.
        const uint32_t koff = lane_off(((16 * ln.w + ln.r) * D + 8 * ln.grp) * 2);
        const uint32_t voff = lane_off(((16 * ln.w + 4 * ln.grp) * D + ln.r * (D / 16)) * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) t.k[ks] = ldb4(kr, koff + 64 * ks);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t off = voff + j * D * 2;
            if constexpr (VW == 4) {
                u32x4 x = ldb4(vr, off);
                t.v[j][0] = x[0]; t.v[j][1] = x[1]; t.v[j][2] = x[2]; t.v[j][3] = x[3];
            } else {
                u32x2 x = ldb2(vr, off);
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

    // Shared-tile path (K and V rows in LDS).  Raw Q K^T of 16 tokens from
    // the lane's KC 16-byte K chunks (chunk i at byte 64 i + 16 grp of its
    // token's row: the d-range of k-step i).
    static constexpr int kRowBytes = D * 2;
    // LDS V row padding: 288-byte rows put the 4 consecutive rows of a
    // transpose read 8 banks apart (4 lanes x 8 bytes per row).
    static constexpr int kVPad = 32;
    static constexpr int KC = D / 32;
    __device__ static f32x4 qk(const u32x4 (&k)[KC], const Q &q) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, k[ks]), __builtin_bit_cast(bf16x8, q.q[ks]), acc,
                0, 0, 0);
        return acc;
    }
    // The lane's D/16 V values of one token (d = r D/16 ..) as bf16 pairs.
    __device__ static void v_row(const uint8_t *row, const Lane &ln, uint32_t (&w)[VW]) {
        const uint8_t *src = row + ln.r * (D / 16) * 2;
        if constexpr (VW == 4) {
            const u32x4 x = *reinterpret_cast<const u32x4 *>(src);
            w[0] = x[0]; w[1] = x[1]; w[2] = x[2]; w[3] = x[3];
        } else {
            const u32x2 x = *reinterpret_cast<const u32x2 *>(src);
            w[0] = x[0]; w[1] = x[1];
        }
    }

    // The V^T operand of d-block blk for the shared-tile path, by two LDS
    // transpose reads of 4 x bf16 each (ds_read_b64_tr_b16): within a group
    // of 16 lanes, lane j receives element j % 4 of the rows that lanes
    // 4 k + j / 4 point at, k = 0 .. 3.  Lane i of k-group g points at token
    // tok(8 g + e), e = 4 h + i / 4 (read h), columns 16 blk + 4 (i % 4) ..,
    // so lane j gets k-slots 8 g .. 8 g + 7 of d = 16 blk + j in k order.
    template <class Tok>
    __device__ static bf16x8 v_tr(const uint8_t *v, int row_bytes, int blk, const Lane &ln,
                                  Tok tok) {
        u32x2 h[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint8_t *a = v + tok(4 * half + (ln.r >> 2)) * row_bytes +
                               2 * (16 * blk + 4 * (ln.r & 3));
            h[half] = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (__attribute__((address_space(3))) v4i16 *)(a)));
        }
        return __builtin_bit_cast(bf16x8, u32x4{h[0][0], h[0][1], h[1][0], h[1][1]});
    }

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

    // K is loaded in whole rows and reordered through the wave's LDS rows.
    static constexpr bool kKRows = true;
    __device__ static void k_operand(uint8_t *rows, const Lane &ln, Tile &t) {
        k_to_operand<D / 16>(rows, ln.lane, ln.r, ln.grp, t.k);
    }

    __device__ static void read_q(const uint32_t *sq, int stride, const Lane &ln, Q &q) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
            q.q[c] = *reinterpret_cast<const u32x4 *>(sq + ln.r * stride + 16 * c + 4 * ln.grp);
    }

    // As for bf16; dead rows read as zero bytes and zero scales.
    __device__ static void load_tile(const DecodeParams &p, int page, int h, int nv,
                                     const Lane &ln, Tile &t) {
        const auto kr = live_rows(p.k, page, h, p.Hkv, D, nv);
        const auto vr = live_rows(p.v, page, h, p.Hkv, D, nv);
        // K in whole rows (k_to_operand reorders them through LDS)
        const uint32_t koff = lane_off(16 * ln.w * D + 16 * ln.lane);
        const uint32_t voff = lane_off((16 * ln.w + 4 * ln.grp) * D + ln.r * (D / 16));
#pragma unroll
        for (int c = 0; c < NC; ++c) t.k[c] = ldb4(kr, koff + 1024 * c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t off = voff + j * D;
            if constexpr (VB == 2) {
                u32x2 x = ldb2(vr, off);
                t.v[j][0] = x[0]; t.v[j][1] = x[1];
            } else {
                t.v[j][0] = ldb1(vr, off);
            }
        }
        // Scales of tokens 16 w + 4 grp + i: one 16-byte run per lane group
        // (the bound is checked per dword).  Waves 2 k and 2 k + 1 read the
        // two halves of one 128-byte line, so these loads keep the default
        // cache policy: with the streaming one the line was often fetched
        // twice (1.5% more HBM reads, 3% more time).
        const uint32_t soff = lane_off((16 * ln.w + 4 * ln.grp) * 4);
        t.ks = __builtin_bit_cast(f32x4,
                                  ldb4_keep(live_rows(p.k_scale, page, h, p.Hkv, 4, nv), soff));
        t.vs = __builtin_bit_cast(f32x4,
                                  ldb4_keep(live_rows(p.v_scale, page, h, p.Hkv, 4, nv), soff));
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

    // Shared-tile path: raw Q K^T of 16 tokens from the lane's KC 16-byte K
    // chunks (chunk c at byte 64 c + 16 grp: k-steps 2 c and 2 c + 1).
    static constexpr int kRowBytes = D;
    // LDS V row padding, as for K rows.
    static constexpr int kVPad = 16;
    static constexpr int KC = D / 64;
    __device__ static f32x4 qk(const u32x4 (&k)[KC], const Q &q) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = ks >> 1, sub = ks & 1;
            const long a = __builtin_bit_cast(long, u32x2{k[c][2 * sub], k[c][2 * sub + 1]});
            const long b = __builtin_bit_cast(long, u32x2{q.q[c][2 * sub], q.q[c][2 * sub + 1]});
            acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, acc, 0, 0, 0);
        }
        return acc;
    }
    // The lane's D/16 V values of one token (d = r D/16 ..) widened to bf16.
    __device__ static void v_row(const uint8_t *row, const Lane &ln, uint32_t (&w)[VW]) {
        const uint8_t *src = row + ln.r * (D / 16);
        uint32_t x[VB];
        if constexpr (VB == 2) {
            const u32x2 y = *reinterpret_cast<const u32x2 *>(src);
            x[0] = y[0]; x[1] = y[1];
        } else {
            x[0] = *reinterpret_cast<const uint32_t *>(src);
        }
#pragma unroll
        for (int c = 0; c < VB; ++c) {
            w[2 * c] = __builtin_bit_cast(uint32_t,
                                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[c], 1.0f, false));
            w[2 * c + 1] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[c], 1.0f, true));
        }
    }

    // The V^T operand of d-block blk for the shared-tile path, by one LDS
    // transpose read of 8 bytes (ds_read_b64_tr_b8): within a group of 16
    // lanes, lane j receives byte j % 8 of the rows that lanes 2 k + j / 8
    // point at, k = 0 .. 7.  Lane i of k-group g points at token
    // tok(8 g + i / 2), bytes 16 blk + 8 (i % 2) .., so lane j gets k-slots
    // 8 g .. 8 g + 7 of d = 16 blk + j in k order, widened here to bf16.
    template <class Tok>
    __device__ static bf16x8 v_tr(const uint8_t *v, int row_bytes, int blk, const Lane &ln,
                                  Tok tok) {
        const uint8_t *a = v + tok(ln.r >> 1) * row_bytes + 16 * blk + 8 * (ln.r & 1);
        const v2i32 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i32 *)(a));
        u32x4 w;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            w[2 * c] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)x[c], 1.0f, false));
            w[2 * c + 1] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)x[c], 1.0f, true));
        }
        return __builtin_bit_cast(bf16x8, w);
    }

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

// A column of the S^T / O^T tiles is held by lanes r, r + 16, r + 32 and
// r + 48 (4 token groups): its max and sum across them.  All lanes.
__device__ __forceinline__ float column_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float column_sum(float x) {
    x += __shfl_xor(x, 16, 64);
    return x + __shfl_xor(x, 32, 64);
}

template <int D, int NCB>
struct State {
    static constexpr int NB = D / 16;   // 16-wide d-blocks of O^T
    f32x4 o[NCB][NB];   // O[column 16 cb + r][d = (4 grp + i) * D/16 + blk]
    // Running max (log2 units) of the column, the same in its 4 lanes, and
    // the running sum of the weights of this lane's tokens: the column's sum
    // is column_sum(l) (the 4 lanes are rescaled by the same factors).
    float m[NCB], l[NCB];

    __device__ void reset() {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
            for (int b = 0; b < NB; ++b) o[cb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
            m[cb] = kNegInf;
            l[cb] = 0.f;
        }
    }
};

// Per-lane constants of the query columns 16 cb + r of a workgroup: column c
// is query row c / G (of R) and head c % G.  A row r sees R - 1 - r fewer
// tokens than the request holds (causal mask among the draft rows).
template <int NCB>
struct Cols {
    int lag[NCB];    // R - 1 - row, 0 for the padding columns c >= R G
    int qoff[NCB];   // row * H_q + head, the column's offset in q_scale
};

// One tile's share for this wave: nv = tokens of the request from the
// tile's first on (live tokens of the tile for nv < 64); the query rows of a
// column see nv - lag of them.
template <class KV, int D, int NCB, bool MR>
__device__ __forceinline__ void attend_tile(const DecodeParams &p, const uint32_t *sq,
                                            const float (&qs)[NCB], const typename KV::Tile &t,
                                            int nv, const Cols<NCB> &cols, State<D, NCB> &st,
                                            const Lane &ln) {
    constexpr int QS = KV::kQRowBytes / 4 + 4;   // LDS Q row stride in dwords
    const int tok0 = 16 * ln.w + 4 * ln.grp;
    s16x4 pb[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        typename KV::Q q;
        KV::read_q(sq + 16 * cb * QS, QS, ln, q);
        f32x4 s = KV::scores(p, q, t, qs[cb], 0, 0, ln);
        if (nv - (rows_per_req<MR>(p) - 1) < kTile) {   // a row sees < 64 of the tile
            const int lim = nv - cols.lag[cb];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tok0 + i >= lim) s[i] = kNegInf;
        }
        float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        // The reference max moves only when a tile's max exceeds it by more
        // than kSlack (log2 units), so weights stay <= 2^kSlack and O, l are
        // rescaled (a wave-uniform branch) only on those rare tiles.  A
        // column's max exceeds the bound iff one of its lanes' maxima does,
        // so the column max is reduced across lanes only on that branch.
        if (__any(mx > st.m[cb] + kSlack)) {
            mx = column_max(mx);
            const bool moves = mx > st.m[cb] + kSlack;
            const float m_new = moves ? mx : st.m[cb];
            // 1 where the reference is kept (also when it stays -inf), 0 from -inf
            const float alpha = moves ? __builtin_amdgcn_exp2f(st.m[cb] - m_new) : 1.f;
            st.l[cb] *= alpha;
#pragma unroll
            for (int b = 0; b < D / 16; ++b) st.o[cb][b] = st.o[cb][b] * alpha;
            st.m[cb] = m_new;
        }
        const float m_use = st.m[cb] == kNegInf ? 0.f : st.m[cb];
        f32x4 pr;
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(s[i] - m_use);
        st.l[cb] += (pr[0] + pr[1]) + (pr[2] + pr[3]);   // this lane's tokens only

        if constexpr (KV::kScaled) pr = pr * t.vs;   // fold the per-token V scale into P
        pb[cb] = __builtin_bit_cast(s16x4,
                                    u32x2{pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3])});
    }

    uint32_t vv[4][D / 32];   // dead rows were loaded as zero
    KV::v_dwords(t, vv);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
        // d-blocks 2c and 2c + 1: low and high bf16 of dword c of each token.
        const u32x2 lo = {halves<false>(vv[0][c], vv[1][c]), halves<false>(vv[2][c], vv[3][c])};
        const u32x2 hi = {halves<true>(vv[0][c], vv[1][c]), halves<true>(vv[2][c], vv[3][c])};
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            st.o[cb][2 * c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(s16x4, lo), pb[cb], st.o[cb][2 * c], 0, 0, 0);
            st.o[cb][2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(s16x4, hi), pb[cb], st.o[cb][2 * c + 1], 0, 0, 0);
        }
    }
}

// LDS scratch for merging the 4 waves of a workgroup, one 16-column block
// at a time (GR = 8 when a workgroup has at most 8 columns).
template <int D, int GR, int NCB, int QW>
struct MergeLds {
    float o[kWaves][GR][D];
    float m[kWaves][GR];
    float l[kWaves][GR];
    // The current descriptor's Q rows of QW words (16 NCB rows, rows >= R G
    // zero), each padded by 4 dwords so that the per-tile operand reads are
    // bank-conflict free.
    alignas(16) uint32_t q[16 * NCB * (QW + 4)];
    int last;   // the fused combine: this workgroup merges the segment
};

// Each wave's 16 padded K rows of RB bytes, on their way to the QK^T
// operand.
template <int RB, bool On = true>
struct KRows {
    alignas(16) uint8_t rows[kWaves][k_rows_bytes<RB / 16>()];
};
template <int RB>
struct KRows<RB, false> {
    uint8_t unused;
};

// This wave's K rows (nullptr where the format needs none).
template <int RB, bool On>
__device__ __forceinline__ uint8_t *k_rows_of(KRows<RB, On> &kr) {
    if constexpr (On)
        return kr.rows[threadIdx.x >> 6];
    else
        return nullptr;
}

// Copy the R G query rows of (b, h) into the LDS Q rows: LDS row r G + g is
// query row r, head h G + g (the G heads of one row are contiguous in q).
// In 16-byte chunks, all loads of a thread issued before its stores: up to
// 16 rows (the per-wave path) that is one chunk per thread, so the staging
// costs one memory round trip per descriptor, not one per pass.  All
// threads.
template <class KV, int D, int GR, int NCB, bool MR, int QW>
__device__ __forceinline__ void stage_q(const DecodeParams &p, MergeLds<D, GR, NCB, QW> &sm, int b,
                                        int h) {
    constexpr int RW = KV::kQRowBytes / 4, QS = RW + 4, CPR = RW / 4;   // CPR chunks per row
    constexpr int NC = (16 * NCB * CPR + kDecodeThreads - 1) / kDecodeThreads;
    const int R = rows_per_req<MR>(p);
    const int n = R * p.G * CPR;
    // the first row of (b, h), wave-uniform; a lane's row r G + g is r H_q + g rows on
    const char *base = reinterpret_cast<const char *>(p.q) +
                       ((int64_t)b * R * p.Hq + (int64_t)h * p.G) * KV::kQRowBytes;
    u32x4 v[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int j = threadIdx.x + i * kDecodeThreads;
        if (j < n) {
            const int row = j / CPR, r = row / p.G, g = row - r * p.G;
            v[i] = ldg<u32x4>(base + (int64_t)r * p.Hq * KV::kQRowBytes,
                              (uint32_t)(g * KV::kQRowBytes + 16 * (j % CPR)));
        }
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int j = threadIdx.x + i * kDecodeThreads;
        if (j < n)
            *reinterpret_cast<u32x4 *>(sm.q + (j / CPR) * QS + 4 * (j % CPR)) = v[i];
    }
}

// ---------------------------------------------------------------------------
// Decode and combine in one launch ("Scheduling around live KV work": the
// partials of a (request, KV head) segment are merged under the global
// softmax once all of them exist).  A segment cut into one chunk writes its
// output directly.  Otherwise every workgroup that finishes one of its
// chunks publishes the partial (agent-scope release) and takes a ticket;
// the one holding the last ticket merges the segment and resets the ticket.
// Nothing waits for another workgroup.
// ---------------------------------------------------------------------------

// Output row of partial row c = r G + g of segment (b, h): out is
// [B, R, H_q, D].
__device__ __forceinline__ int64_t out_row(const DecodeParams &p, int b, int h, int c) {
    return ((int64_t)b * p.R + c / p.G) * p.Hq + (int64_t)h * p.G + c % p.G;
}

__device__ __forceinline__ void store_bf16x4(void *out, int64_t elem, const f32x4 &v) {
    const u32x2 w = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    *reinterpret_cast<u32x2 *>(reinterpret_cast<__bf16 *>(out) + elem) = w;
}

// Partials that another workgroup merges are written and read with the
// device-coherent cache policy (sc1: the L2 of another XCD cannot hold a
// stale copy), through buffer descriptors based at the rows concerned, so
// that no release / acquire fence (a write-back or invalidate of the whole
// L2 of an XCD) is needed around the ticket.  Out-of-range offsets read 0
// and write nothing.
constexpr int kCoherent = 16;          // cache policy: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const float *base, int64_t floats) {
    return span_rsrc(base, (int)(floats * 4));
}

__device__ __forceinline__ void publish4(__amdgpu_buffer_rsrc_t r, uint32_t byte, const f32x4 &v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)byte, 0,
                                           kCoherent);
}

__device__ __forceinline__ void publish(__amdgpu_buffer_rsrc_t r, uint32_t byte, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)byte, 0, kCoherent);
}

__device__ __forceinline__ f32x4 fetch4(__amdgpu_buffer_rsrc_t r, uint32_t byte) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte, 0,
                                                                         kCoherent));
}

__device__ __forceinline__ float fetch(__amdgpu_buffer_rsrc_t r, uint32_t byte) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)byte, 0, kCoherent));
}

// Merge the n partials k0 .. k0 + n - 1 of segment (b, h) into out / out_lse
// (all threads of the workgroup; lse is natural log, -inf for no weight).
// One pass with a running maximum, kMergeUnroll chunks' loads in flight.
constexpr int kMergeUnroll = 4;

template <int D>
__device__ __forceinline__ void merge_segment(const DecodeParams &p, int b, int h, int64_t k0,
                                              int n, int nthreads) {
    const int RG = p.R * p.G;
    const auto ro = rows_rsrc(p.part_o + k0 * RG * D, (int64_t)n * RG * D);
    const auto rl = rows_rsrc(p.part_lse + k0 * RG, (int64_t)n * RG);
    for (int e = 4 * threadIdx.x; e < RG * D; e += 4 * nthreads) {
        const int c = e / D, d = e % D;
        float M = kNegInf, W = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < n; k += kMergeUnroll) {
            float l[kMergeUnroll];
            f32x4 o[kMergeUnroll];
#pragma unroll
            for (int u = 0; u < kMergeUnroll; ++u) {   // past n: no weight (o reads 0)
                const int kk = k + u;
                l[u] = kk < n ? fetch(rl, 4u * (uint32_t)(kk * RG + c)) : kNegInf;
                o[u] = fetch4(ro, 4u * (uint32_t)((kk * RG + c) * D + d));
            }
#pragma unroll
            for (int u = 0; u < kMergeUnroll; ++u) {
                if (l[u] == kNegInf) continue;
                const float M2 = fmaxf(M, l[u]);
                const float a = __expf(M - M2), w = __expf(l[u] - M2);   // M = -inf: a = 0
                W = W * a + w;
                acc = acc * a + w * o[u];
                M = M2;
            }
        }
        if (M != kNegInf) acc = acc * (1.0f / W);
        const int64_t row = out_row(p, b, h, c);
        store_bf16x4(p.out, row * D + d, acc);
        if (p.out_lse && d == 0) p.out_lse[row] = M == kNegInf ? kNegInf : M + __logf(W);
    }
}

// After a workgroup wrote the partial of its descriptor in segment (b, h)
// (all threads): take a ticket; the last one merges.  `last` is LDS.
//
// Why the last workgroup sees every partial, on a chip whose 8 XCDs each
// have an L2 that is not coherent with the others, without the release /
// acquire fences of the language (each would write back or invalidate a
// whole L2):
//   1. every partial row and LSE is stored with the sc1 cache policy
//      (publish4 / publish), which writes through the XCD's L2 to the
//      device-coherent level;
//   2. each wave waits until its stores are acknowledged (s_waitcnt
//      vmcnt(0): on gfx950 stores count in vmcnt, and an sc1 store is
//      acknowledged once it is device-coherent), then the barrier orders
//      all waves of the workgroup before the ticket;
//   3. the ticket is an agent-scope atomic, performed at the device-coherent
//      level, so every workgroup's increment is ordered after its own
//      partials became device-coherent;
//   4. the workgroup that takes the last ticket loads the partials with sc1
//      (fetch4 / fetch): they miss its own L2 and read the device-coherent
//      copies.  Those loads are issued only after the atomic returned and
//      the barrier that broadcasts `last`, so none can precede it.
// The reset is an agent-scope atomic store too, so the next launch (or the
// next call on the same tickets) reads zero without relying on the L2
// write-back at the end of this kernel.
template <int D>
__device__ __forceinline__ void ticket_and_merge(const DecodeParams &p, int b, int h,
                                                 int64_t k0, int n, int &last, int nthreads) {
    const int s = b * p.Hkv + h;
    // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15): this wave's partial stores
    // are device-coherent before the barrier and the ticket.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (threadIdx.x == 0)
        last = __hip_atomic_fetch_add(p.tickets + s, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == n - 1;
    __syncthreads();
    if (last) {
        merge_segment<D>(p, b, h, k0, n, nthreads);
        if (threadIdx.x == 0)
            __hip_atomic_store(p.tickets + s, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Segments with no chunk (an empty request) get out = 0, lse = -inf from
// workgroup s mod P, before its bin (all threads).
template <int D>
__device__ __forceinline__ void clear_empty_segments(const DecodeParams &p, int nthreads) {
    const MapLayout lay(p.B, p.Hkv, p.P);
    const int S = p.B * p.Hkv, RG = p.R * p.G;
    for (int s = blockIdx.x; s < S; s += p.P) {
        if (sload(p.map + lay.seg_off, s + 1) != sload(p.map + lay.seg_off, s)) continue;
        const int b = s / p.Hkv, h = s % p.Hkv;
        for (int e = 4 * threadIdx.x; e < RG * D; e += 4 * nthreads) {
            const int c = e / D, d = e % D;
            const int64_t row = out_row(p, b, h, c);
            store_bf16x4(p.out, row * D + d, f32x4{0.f, 0.f, 0.f, 0.f});
            if (p.out_lse && d == 0) p.out_lse[row] = kNegInf;
        }
    }
}

// The chunk count of segment (b, h) and its first partial slot, when the
// combine is fused (n = 0 otherwise).
template <bool FU>
__device__ __forceinline__ int seg_chunks(const DecodeParams &p, int b, int h, int64_t &k0) {
    k0 = 0;
    if constexpr (!FU) return 0;
    const MapLayout lay(p.B, p.Hkv, p.P);
    const int s = b * p.Hkv + h;
    k0 = sload(p.map + lay.seg_off, s);
    return sload(p.map + lay.seg_off, s + 1) - (int)k0;
}

// Merge the waves' states and write partial slot `slot` (R G rows).  All
// threads.
template <int D, int GR, int NCB, bool MR, bool FU, class Between, int QW>
__device__ __forceinline__ void merge_write(const DecodeParams &p, State<D, NCB> &st,
                                            MergeLds<D, GR, NCB, QW> &sm, int64_t slot, int b, int h,
                                            const Lane &ln, Between between) {
    const int RG = rows_per_req<MR>(p) * p.G;
    int64_t k0;
    const int nch = seg_chunks<FU>(p, b, h, k0);   // fused combine: where the rows go
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int c0 = 16 * cb;
        const float lsum = column_sum(st.l[cb]);
        if (c0 + ln.r < RG) {
            if (ln.grp == 0) {
                sm.m[ln.w][ln.r] = st.m[cb];
                sm.l[ln.w][ln.r] = lsum;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float *dst = &sm.o[ln.w][ln.r][(4 * ln.grp + i) * (D / 16)];
#pragma unroll
                for (int blk = 0; blk < D / 16; blk += 4)
                    *reinterpret_cast<f32x4 *>(dst + blk) =
                        f32x4{st.o[cb][blk][i], st.o[cb][blk + 1][i], st.o[cb][blk + 2][i],
                              st.o[cb][blk + 3][i]};
            }
        }
        __syncthreads();
        const int n = min(16, RG - c0);
        for (int e = 4 * threadIdx.x; e < n * D; e += 4 * kDecodeThreads) {
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
            const float lse = M == kNegInf ? kNegInf : (M + log2f(wsum)) * kLn2;
            if (nch == 1) {   // the segment's only chunk: its partial is the output
                const int64_t row = out_row(p, b, h, c0 + g);
                store_bf16x4(p.out, row * D + d, acc);
                if (p.out_lse && d == 0) p.out_lse[row] = lse;
                continue;
            }
            // the slot's rows start at a uniform address, plus a 32-bit offset
            char *obase = reinterpret_cast<char *>(p.part_o + slot * RG * D);
            float *dst = reinterpret_cast<float *>(obase + 4u * (uint32_t)((c0 + g) * D + d));
            if constexpr (FU) {   // merged by another workgroup
                publish4(rows_rsrc(p.part_o + slot * RG * D, (int64_t)RG * D),
                         4u * (uint32_t)((c0 + g) * D + d), acc);
                if (d == 0)
                    publish(rows_rsrc(p.part_lse + slot * RG, RG), 4u * (uint32_t)(c0 + g), lse);
            } else {
                *reinterpret_cast<f32x4 *>(dst) = acc;
                if (d == 0) p.part_lse[slot * RG + c0 + g] = lse;
            }
        }
        if (cb + 1 < NCB) __syncthreads();   // the next block reuses sm.o
    }
    if constexpr (FU)
        if (nch > 1) ticket_and_merge<D>(p, b, h, k0, nch, sm.last, kDecodeThreads);
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
        const int64_t o = 4 * (int64_t)d;
        const int b = sload(desc, o);
        return Pos{d, b, sload(desc, o + 1), sload(desc, o + 2), sload(desc, o + 3), sload(lens, b)};
    }
};

// The walk with the next descriptor read ahead: `pre` is the first tile of
// descriptor x.d + 1, read when descriptor x.d was entered, so that crossing
// a descriptor boundary waits for no descriptor read (only the page id).
// Past the run's last descriptor it repeats that one (a valid read); runs
// without a map (the static kernel) have a single range and read nothing.
__device__ __forceinline__ Pos read_ahead(const MapSource &src, int d_end, const Pos &x) {
    return src.desc ? src.read(min(x.d + 1, d_end - 1)) : x;
}

__device__ __forceinline__ bool advance_ahead(int d_end, const Pos &x, const Pos &pre, Pos &y) {
    const bool same = x.t + 1 < x.t1;
    Pos n = x;
    n.t = x.t + 1;
    y = pick(same, n, pre);
    return same || x.d + 1 < d_end;
}

// Page id of the tile at x and the request's tokens from the tile's first
// on (nv, not clamped to 64: a query row that sees lag fewer tokens than the
// request holds needs nv - lag); a tile outside the page table or with a
// page id outside the pool reads page 0 and counts no token.
__device__ __forceinline__ int locate(const DecodeParams &p, const Pos &x, int &nv) {
    nv = x.L - kTile * x.t;
    int page = x.t < p.max_pages ? sload(p.page_table, (int64_t)x.b * p.max_pages + x.t) : -1;
    if ((unsigned)page >= (unsigned)p.num_pages) {
        page = 0;
        nv = 0;
    }
    return page;
}

// fp8: the q_scale of each of this lane's columns of (x.b, x.h); 1 for bf16.
template <class KV, int NCB, bool MR>
__device__ __forceinline__ void q_scale_of(const DecodeParams &p, const Pos &x,
                                           const Cols<NCB> &cols, float (&qs)[NCB]) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        if constexpr (KV::kScaled)
            qs[cb] = p.q_scale[(int64_t)x.b * rows_per_req<MR>(p) * p.Hq + (int64_t)x.h * p.G +
                               cols.qoff[cb]];
        else
            qs[cb] = 1.f;
    }
}

template <int NCB, bool MR>
__device__ __forceinline__ Cols<NCB> columns(const DecodeParams &p, const Lane &ln) {
    Cols<NCB> c;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int col = 16 * cb + ln.r;
        if constexpr (MR) {
            const bool real = col < p.R * p.G;
            const int row = real ? col / p.G : 0;
            c.lag[cb] = real ? p.R - 1 - row : 0;
            c.qoff[cb] = real ? row * p.Hq + col % p.G : 0;
        } else {
            c.lag[cb] = 0;
            c.qoff[cb] = col < p.G ? col : 0;
        }
    }
    return c;
}

// Wave priority from a bin's progress.  The SIMDs issue the oldest wave
// first, so among the equal bins of one CU the workgroup that arrived first
// finishes first and the last one runs its tail alone, on a fraction of the
// CU's issue slots.  That tail costs the compute-heavy multi-row kernels a
// few percent; the one-row kernel gains 1% on mixed lengths from evening it
// out and loses 0.5% on a few long requests among many short.  A wave starts at
// priority 3 and steps down by one after each quarter of q tiles (the size
// of every bin, within one tile), so the waves that are behind issue first
// and the bins of a CU end together.  All counters are wave-uniform, and
// s_setprio takes an immediate.
struct Fairness {
    int quarter, left, level;
    __device__ explicit Fairness(int q_tiles)
        : quarter(max(1, q_tiles >> 2)), left(max(1, q_tiles >> 2)), level(3) {}
    __device__ void start() const { __builtin_amdgcn_s_setprio(3); }
    __device__ void tile() {
        if (--left > 0 || level == 0) return;
        left = quarter;
        if (--level == 2)
            __builtin_amdgcn_s_setprio(2);
        else if (level == 1)
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
    }
};

// Drains a run of descriptors tile by tile: while tile i is computed, tile
// i + 1 (across descriptor boundaries) is being loaded into the other
// register buffer.  The run starts at `first` and ends with descriptor
// d_end - 1; partials go to slot d (by_desc) or to slot_base.
template <class KV, int D, int GR, int NCB, bool MR, bool FU, int QW>
__device__ __forceinline__ void drain(const DecodeParams &p, MergeLds<D, GR, NCB, QW> &sm,
                                      uint8_t *krows, const MapSource &src, const Pos &first,
                                      int d_end, int64_t slot_base, bool by_desc) {
    using Tile = typename KV::Tile;
    const Lane ln;
    const Cols<NCB> cols = columns<NCB, MR>(p, ln);
    State<D, NCB> st;
    Pos cur = first;
    int nv_cur;

    // Q rows past R G stay zero for the whole kernel.
    for (int i = threadIdx.x; i < (int)(sizeof(sm.q) / 4); i += kDecodeThreads) sm.q[i] = 0u;
    __syncthreads();
    stage_q<KV, D, GR, NCB, MR>(p, sm, cur.b, cur.h);
    float qs[NCB];
    q_scale_of<KV, NCB, MR>(p, cur, cols, qs);
    st.reset();
    Pos pre = read_ahead(src, d_end, cur);
    Tile ta, tb;
    const int pg = locate(p, cur, nv_cur);
    KV::load_tile(p, pg, cur.h, nv_cur, ln, ta);
    __syncthreads();
    Fairness fair(by_desc ? sload(p.map, 2) : 1 << 30);   // bins of q tiles (map word 2)
    if (by_desc) fair.start();

    // Issue tile i + 1 into `nxt` (after the last tile, a load of no rows,
    // which touches no memory and keeps the steady-state path branch-free),
    // compute tile i from `now`, close its descriptor if it ends, staging
    // the next descriptor's Q in LDS inside the merge's barriers.
    auto step = [&](Tile &now, Tile &nxt) __attribute__((always_inline)) -> bool {
        Pos n;
        const bool more = advance_ahead(d_end, cur, pre, n);
        const Pos far = pick(more, n, cur);
        int nv_n;
        const int pg_n = locate(p, far, nv_n);
        KV::load_tile(p, pg_n, far.h, more ? nv_n : 0, ln, nxt);

        if (by_desc) fair.tile();
        KV::k_operand(krows, ln, now);
        attend_tile<KV, D, NCB, MR>(p, sm.q, qs, now, nv_cur, cols, st, ln);

        if (!more || n.d != cur.d) {
            merge_write<D, GR, NCB, MR, FU>(p, st, sm, by_desc ? (int64_t)cur.d : slot_base, cur.b,
                                        cur.h, ln,
                                        [&] {
                                            if (more) stage_q<KV, D, GR, NCB, MR>(p, sm, n.b, n.h);
                                        });
            if (!more) return false;
            pre = read_ahead(src, d_end, n);
            q_scale_of<KV, NCB, MR>(p, n, cols, qs);
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

// ---------------------------------------------------------------------------
// The shared-tile path, for 2 .. 4 column blocks (multi-row steps with
// R G > 16).  Holding every column's O in every wave (the path above) would
// need NCB x D/4 accumulator registers per lane.  Here a workgroup is NCB
// compute waves, wave w owns column block w for all 64 tokens of a tile, and
// the tile sits in LDS, read by every column block:
//   * the next tile is copied from HBM into registers (16-byte nontemporal
//     loads) while the waves compute the current one from LDS, by all
//     threads or, for three column blocks at D = 128, by a fourth wave that
//     only stages (drain_shared_staged);
//   * a barrier, the registers go to LDS (K rows padded by 16 bytes, so that
//     16 lanes reading 16 rows at one column hit distinct banks; bf16 V
//     rows by 32, for the transpose reads), a barrier;
//   * S^T = K Q^T per 16-token block on v_mfma_f32_16x16x32_{bf16,fp8};
//     O^T += V^T P^T over 32 tokens per v_mfma_f32_16x16x32_bf16 (the lane's
//     tokens of two 16-token blocks form its 8 k-slots);
//   * a wave has its columns' whole softmax state, so a descriptor's partial
//     is written without a merge between waves;
//   * with the combine fused, the compute waves also take the segment's
//     ticket and the last workgroup's compute waves merge it; a staging
//     wave only joins the ticket's barriers.
// ---------------------------------------------------------------------------

template <class KV, int D>
struct SharedLds {
    static constexpr int kRow = KV::kRowBytes + 16;           // padded K row
    static constexpr int kRowV = KV::kRowBytes + KV::kVPad;   // padded V row
    alignas(16) uint8_t kv[kTile * (kRow + kRowV)];   // K rows 0 .. 63, then V rows
    alignas(16) float ks[kTile];   // fp8 k and v scales of the tile's tokens
    alignas(16) float vs[kTile];
    int last;   // the fused combine: this workgroup merges the segment
    __device__ const uint8_t *k() const { return kv; }
    __device__ const uint8_t *v() const { return kv + kTile * kRow; }
    __device__ uint8_t *v() { return kv + kTile * kRow; }
};

// The tile as 16-byte chunks: K rows (chunk j < NK), V rows, then for fp8
// the 16 chunks of k scales at 2 NK and the 16 of v scales at 2 NK + 64.
// Staging thread t of T (all threads of the workgroup, or the 64 of its
// staging wave) moves chunks t, t + T, ...  NK and T are multiples of 64,
// so a wave's 64 chunks of a round are all K, all V, or one kind of scale:
// the choice of source is wave-uniform.
template <class KV, int D, int T_>
struct Staged {
    static constexpr int T = T_;
    static constexpr int NK = kTile * KV::kRowBytes / 16;
    static constexpr int KSC = 2 * NK, VSC = 2 * NK + 64;   // first scale chunks
    static constexpr int NT = KV::kScaled ? VSC + 16 : 2 * NK;
    static constexpr int NCH = (NT + T - 1) / T;
    static_assert(NK % 64 == 0, "K and V rounds split at wave boundaries");
    u32x4 c[NCH];
};

// The first chunk of staging thread tid's wave in round i (wave-uniform).
template <class S>
__device__ __forceinline__ int wave_chunk0(int i, int tid) {
    return S::T * i + 64 * __builtin_amdgcn_readfirstlane(tid >> 6);
}

template <class KV, int D, int T>
__device__ __forceinline__ void stage_load(const DecodeParams &p, int page, int h, int nv,
                                           Staged<KV, D, T> &st, int tid) {
    using S = Staged<KV, D, T>;
    // Dead rows (token >= nv) and their scales read as zero.
    const auto kr = live_rows(p.k, page, h, p.Hkv, KV::kRowBytes, nv);
    const auto vr = live_rows(p.v, page, h, p.Hkv, KV::kRowBytes, nv);
    const int lane = tid & 63;
#pragma unroll
    for (int i = 0; i < S::NCH; ++i) {
        const int j = tid + S::T * i;
        if (S::T * (i + 1) <= S::NK) {   // all K (a whole round of chunks)
            st.c[i] = ldb4(kr, 16 * j);
        } else if (S::T * i >= S::NK && S::T * (i + 1) <= 2 * S::NK) {   // all V
            st.c[i] = ldb4(vr, 16 * (j - S::NK));
        } else {   // a round across K, V and the scales: one source per wave
            const int j0 = wave_chunk0<S>(i, tid);
            if (j0 < S::NK) {
                st.c[i] = ldb4(kr, 16 * j);
            } else if (j0 < 2 * S::NK) {
                st.c[i] = ldb4(vr, 16 * (j - S::NK));
            } else if constexpr (KV::kScaled) {
                if (j0 == S::KSC && lane < 16)
                    st.c[i] = ldb4(live_rows(p.k_scale, page, h, p.Hkv, 4, nv), 16 * lane);
                else if (j0 == S::VSC && lane < 16)
                    st.c[i] = ldb4(live_rows(p.v_scale, page, h, p.Hkv, 4, nv), 16 * lane);
            }
        }
    }
}

// K and V chunks go to row j / CPR, column j % CPR of the K-then-V rows
// (CPR chunks per row); a round of T threads covers T / CPR whole rows, so
// the address of round i is the thread's first address plus a constant.
template <class KV, int D, int T>
__device__ __forceinline__ void stage_store(SharedLds<KV, D> &sm, const Staged<KV, D, T> &st,
                                            int tid) {
    using S = Staged<KV, D, T>;
    using L = SharedLds<KV, D>;
    constexpr int CPR = KV::kRowBytes / 16;
    static_assert(S::T % CPR == 0, "a round of chunks covers whole rows");
    uint8_t *kbase = sm.kv + (tid / CPR) * L::kRow + 16 * (tid % CPR);
    // V chunk of round i: row tid / CPR + (T / CPR) i - 64, column tid % CPR
    uint8_t *vbase = sm.v() + (tid / CPR - kTile) * L::kRowV + 16 * (tid % CPR);
#pragma unroll
    for (int i = 0; i < S::NCH; ++i) {
        const int j = tid + S::T * i;
        if (S::T * (i + 1) <= S::NK) {   // a whole round of K chunks
            *reinterpret_cast<u32x4 *>(kbase + (S::T / CPR) * L::kRow * i) = st.c[i];
        } else if (S::T * i >= S::NK && S::T * (i + 1) <= 2 * S::NK) {   // of V chunks
            *reinterpret_cast<u32x4 *>(vbase + (S::T / CPR) * L::kRowV * i) = st.c[i];
        } else if (j < S::NK) {
            *reinterpret_cast<u32x4 *>(kbase + (S::T / CPR) * L::kRow * i) = st.c[i];
        } else if (j < 2 * S::NK) {
            *reinterpret_cast<u32x4 *>(vbase + (S::T / CPR) * L::kRowV * i) = st.c[i];
        } else if (KV::kScaled && j >= S::KSC && j < S::KSC + 16) {
            *reinterpret_cast<u32x4 *>(sm.ks + 4 * (j - S::KSC)) = st.c[i];
        } else if (KV::kScaled && j >= S::VSC && j < S::VSC + 16) {
            *reinterpret_cast<u32x4 *>(sm.vs + 4 * (j - S::VSC)) = st.c[i];
        }
    }
}

// One tile from LDS for the 16 columns of this wave's block, in two halves
// of 32 tokens (token blocks 2 th, 2 th + 1), each folded into the running
// softmax state on its own.  nv as in attend_tile; lag and qs are this
// lane's column's.
template <class KV, int D>
__device__ __forceinline__ void attend_shared(const DecodeParams &p, const SharedLds<KV, D> &sm,
                                              const typename KV::Q &q, float qs, int nv, int lag,
                                              State<D, 1> &st, const Lane &ln) {
    constexpr int kRow = SharedLds<KV, D>::kRow, kRowV = SharedLds<KV, D>::kRowV;
    const bool masked = nv - (p.R - 1) < 2 * 32;   // some row sees < 64 tokens
    const int lim = nv - lag;
#pragma unroll
    for (int th = 0; th < 2; ++th) {
        f32x4 s[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {   // 16-token blocks tb = 2 th + u
            const int tb = 2 * th + u;
            u32x4 kc[KV::KC];
            const uint8_t *row = sm.k() + (16 * tb + ln.r) * kRow + 16 * ln.grp;
#pragma unroll
            for (int i = 0; i < KV::KC; ++i) kc[i] = *reinterpret_cast<const u32x4 *>(row + 64 * i);
            s[u] = KV::qk(kc, q);
            if constexpr (KV::kScaled)
                s[u] = s[u] * *reinterpret_cast<const f32x4 *>(sm.ks + 16 * tb + 4 * ln.grp) *
                       (qs * p.scale_log2);
            else
                s[u] = s[u] * p.scale_log2;
            if (masked) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * tb + 4 * ln.grp + i >= lim) s[u][i] = kNegInf;
            }
        }
        float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        if (__any(mx > st.m[0] + kSlack)) {   // stale reference max, as in attend_tile
            mx = column_max(mx);
            const bool moves = mx > st.m[0] + kSlack;
            const float m_new = moves ? mx : st.m[0];
            const float alpha = moves ? __builtin_amdgcn_exp2f(st.m[0] - m_new) : 1.f;
            st.l[0] *= alpha;
#pragma unroll
            for (int b = 0; b < D / 16; ++b) st.o[0][b] = st.o[0][b] * alpha;
            st.m[0] = m_new;
        }
        const float m_use = st.m[0] == kNegInf ? 0.f : st.m[0];
        float ps = 0.f;
        uint32_t pw[4];   // P of tokens 32 th + 16 u + 4 grp + i, bf16 pairs
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 pr;
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(s[u][i] - m_use);
            ps += (pr[0] + pr[1]) + (pr[2] + pr[3]);
            if constexpr (KV::kScaled)
                pr = pr * *reinterpret_cast<const f32x4 *>(sm.vs + 32 * th + 16 * u + 4 * ln.grp);
            pw[2 * u] = pack_bf16(pr[0], pr[1]);
            pw[2 * u + 1] = pack_bf16(pr[2], pr[3]);
        }
        st.l[0] += ps;   // this lane's tokens only

        // O^T += V^T P^T over the half's 32 tokens: k-slot e < 4 of k-group
        // g is token 32 th + 4 g + e, e >= 4 token 32 th + 16 + 4 g + e - 4
        // (where the lane's P values sit); d-block blk covers d = 16 blk ..
        // 16 blk + 15 (O^T row m is d = 16 blk + m).  Dead V rows are zero.
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
        const auto tok = [&](int e) { return 32 * th + 16 * (e >> 2) + 4 * ln.grp + (e & 3); };
#pragma unroll
        for (int blk = 0; blk < D / 16; ++blk)
            st.o[0][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                KV::v_tr(sm.v(), kRowV, blk, ln, tok), pb, st.o[0][blk], 0, 0, 0);
    }
}

// Normalise and write this wave's columns of partial slot `slot` of
// segment (b, h), which has nch chunks when the combine is fused: the only
// chunk of a segment writes the output rows directly, and a chunk that
// another workgroup may merge is published device-coherent.  The slot's
// rows start at a uniform address; the lane adds a 32-bit offset.
template <int D, bool FU>
__device__ __forceinline__ void write_columns(const DecodeParams &p, const State<D, 1> &st,
                                              int col0, int64_t slot, int b, int h, int nch,
                                              const Lane &ln) {
    const int RG = p.R * p.G;
    const int col = col0 + ln.r;
    const float l = column_sum(st.l[0]);
    if (col >= RG) return;
    const bool live = l > 0.f;
    const float inv = live ? 1.0f / l : 0.f;
    const float lse = live ? (st.m[0] + log2f(l)) * kLn2 : kNegInf;
    // accumulator blk holds d = 16 blk + 4 grp .. 16 blk + 4 grp + 3
    if (FU && nch == 1) {
        const int64_t row = out_row(p, b, h, col);
#pragma unroll
        for (int blk = 0; blk < D / 16; ++blk)
            store_bf16x4(p.out, row * D + 16 * blk + 4 * ln.grp, st.o[0][blk] * inv);
        if (p.out_lse && ln.grp == 0) p.out_lse[row] = lse;
        return;
    }
    if constexpr (FU) {
        const auto ro = rows_rsrc(p.part_o + slot * RG * D, (int64_t)RG * D);
#pragma unroll
        for (int blk = 0; blk < D / 16; ++blk)
            publish4(ro, 4u * (uint32_t)(col * D + 16 * blk + 4 * ln.grp), st.o[0][blk] * inv);
        if (ln.grp == 0) publish(rows_rsrc(p.part_lse + slot * RG, RG), 4u * (uint32_t)col, lse);
    } else {
        char *obase = reinterpret_cast<char *>(p.part_o + slot * RG * D);
#pragma unroll
        for (int blk = 0; blk < D / 16; ++blk)
            *reinterpret_cast<f32x4 *>(obase + (uint32_t)(col * D + 16 * blk + 4 * ln.grp) * 4u) =
                st.o[0][blk] * inv;
        if (ln.grp == 0) p.part_lse[slot * RG + col] = lse;
    }
}

// The end of descriptor `slot` in segment (b, h) on the shared-tile path:
// every compute wave writes its columns; with the combine fused, a segment
// of several chunks then takes a ticket and its last workgroup merges it
// (the compute waves, nthreads threads; a staging wave takes the two
// barriers of the ticket with them, in ticket_barriers).
template <int D, bool FU>
__device__ __forceinline__ void close_descriptor(const DecodeParams &p, const State<D, 1> &st,
                                                 int &last, int64_t slot, int b, int h,
                                                 const Lane &ln, int nthreads) {
    int64_t k0;
    const int nch = seg_chunks<FU>(p, b, h, k0);
    write_columns<D, FU>(p, st, 16 * ln.w, slot, b, h, nch, ln);
    if constexpr (FU)
        if (nch > 1) ticket_and_merge<D>(p, b, h, k0, nch, last, nthreads);
}

// The staging wave's share of close_descriptor: the ticket's two barriers
// when the segment has more than one chunk.
template <bool FU>
__device__ __forceinline__ void ticket_barriers(const DecodeParams &p, int b, int h) {
    if constexpr (FU) {
        int64_t k0;
        if (seg_chunks<FU>(p, b, h, k0) > 1) {
            __syncthreads();
            __syncthreads();
        }
    }
}

// This lane's column of the shared-tile path: its query row's lag, its
// q_scale offset and its Q row's offset in q (columns past R G read none).
struct SharedCol {
    bool real;
    int lag, qoff;
    __device__ SharedCol(const DecodeParams &p, const Lane &ln) {
        const int col = 16 * ln.w + ln.r;
        real = col < p.R * p.G;
        const int qrow = real ? col / p.G : 0;
        lag = real ? p.R - 1 - qrow : 0;
        qoff = real ? qrow * p.Hq + col % p.G : 0;
    }
};

// The lane's Q operand of (x.b, x.h), straight from q: the same d-ranges as
// the K chunks (chunk i at byte 64 i + 16 grp of the row); zero for columns
// past R G.
template <class KV>
__device__ __forceinline__ void load_q_direct(const DecodeParams &p, const Pos &x,
                                              const SharedCol &c, const Lane &ln,
                                              typename KV::Q &q) {
    const char *base = reinterpret_cast<const char *>(p.q) +
                       ((int64_t)x.b * p.R * p.Hq + (int64_t)x.h * p.G) * KV::kQRowBytes;
    const uint32_t off = (uint32_t)(c.qoff * KV::kQRowBytes + 16 * ln.grp);
#pragma unroll
    for (int i = 0; i < KV::kQRowBytes / 64; ++i)
        q.q[i] = c.real ? ldg<u32x4>(base, off + 64 * i) : u32x4{0u, 0u, 0u, 0u};
}

// The drain loop of the shared-tile path (same descriptor walk as drain):
// tile t + 1 is issued into registers before tile t is computed from LDS
// and stored to LDS after it.
template <class KV, int D, int NCB, bool FU>
__device__ __forceinline__ void drain_shared(const DecodeParams &p, SharedLds<KV, D> &sm,
                                             const MapSource &src, const Pos &first, int d_end,
                                             int64_t slot_base, bool by_desc) {
    const Lane ln;
    const SharedCol col(p, ln);
    auto q_scale_at = [&](const Pos &x) __attribute__((always_inline)) -> float {
        if constexpr (KV::kScaled)
            return ldg<float>(p.q_scale + ((int64_t)x.b * p.R * p.Hq + (int64_t)x.h * p.G),
                              (uint32_t)col.qoff * 4u);
        else
            return 1.f;
    };

    State<D, 1> st;
    typename KV::Q q;
    Pos cur = first;
    int nv_cur;
    Pos pre = read_ahead(src, d_end, cur);
    Staged<KV, D, 64 * NCB> stg;
    const int tid = threadIdx.x;
    {
        const int pg = locate(p, cur, nv_cur);
        stage_load<KV, D, 64 * NCB>(p, pg, cur.h, nv_cur, stg, tid);
    }
    load_q_direct<KV>(p, cur, col, ln, q);
    float qs = q_scale_at(cur);
    st.reset();
    stage_store<KV, D, 64 * NCB>(sm, stg, tid);
    __syncthreads();
    // The dynamic kernel's bins hold q tiles each (header word 2 of the map).
    Fairness fair(by_desc ? sload(p.map, 2) : 1 << 30);
    if (by_desc) fair.start();

    while (true) {
        Pos n;
        const bool more = advance_ahead(d_end, cur, pre, n);
        const Pos far = pick(more, n, cur);
        int nv_n;
        const int pg_n = locate(p, far, nv_n);
        stage_load<KV, D, 64 * NCB>(p, pg_n, far.h, more ? nv_n : 0, stg, tid);

        if (by_desc) fair.tile();
        attend_shared<KV, D>(p, sm, q, qs, nv_cur, col.lag, st, ln);
        __syncthreads();   // every wave is done with the tile in LDS

        if (!more || n.d != cur.d) {
            close_descriptor<D, FU>(p, st, sm.last, by_desc ? (int64_t)cur.d : slot_base, cur.b,
                                    cur.h, ln, 64 * NCB);
            if (!more) return;
            pre = read_ahead(src, d_end, n);
            load_q_direct<KV>(p, n, col, ln, q);
            qs = q_scale_at(n);
            st.reset();
        }
        stage_store<KV, D, 64 * NCB>(sm, stg, tid);
        __syncthreads();   // tile t + 1 is in LDS
        cur = n;
        nv_cur = nv_n;
    }
}

// The same walk with a staging wave: waves 0 .. NCB - 1 compute from LDS
// and wave NCB alone copies tile t + 1 HBM -> registers -> LDS.  Nothing
// that one kind of wave holds is live in the other's loop, so the staging
// wave's 2 NK / 64 chunks per lane and the compute waves' accumulators do
// not add up.  Both loops take the same barriers: one when the tile in LDS
// is no longer read, one when the next tile is in.
template <class KV, int D, int NCB, bool FU>
__device__ __forceinline__ void drain_shared_staged(const DecodeParams &p, SharedLds<KV, D> &sm,
                                                    const MapSource &src, const Pos &first,
                                                    int d_end, int64_t slot_base, bool by_desc) {
    const Lane ln;
    Pos cur = first;
    Pos pre = read_ahead(src, d_end, cur);
    if (uniform(ln.w) == NCB) {
        __builtin_amdgcn_s_setprio(3);   // its loads and stores go first
        Staged<KV, D, 64> stg;
        int nv;
        const int pg = locate(p, cur, nv);
        stage_load<KV, D, 64>(p, pg, cur.h, nv, stg, ln.lane);
        stage_store<KV, D, 64>(sm, stg, ln.lane);
        __syncthreads();
        while (true) {
            Pos n;
            const bool more = advance_ahead(d_end, cur, pre, n);
            const Pos far = pick(more, n, cur);
            int nv_n;
            const int pg_n = locate(p, far, nv_n);
            stage_load<KV, D, 64>(p, pg_n, far.h, more ? nv_n : 0, stg, ln.lane);
            __syncthreads();   // every compute wave is done with the tile in LDS
            if (!more || n.d != cur.d) ticket_barriers<FU>(p, cur.b, cur.h);
            if (!more) return;
            if (n.d != cur.d) pre = read_ahead(src, d_end, n);
            stage_store<KV, D, 64>(sm, stg, ln.lane);
            __syncthreads();   // tile t + 1 is in LDS
            cur = n;
        }
    }

    const SharedCol col(p, ln);
    auto q_scale_at = [&](const Pos &x) __attribute__((always_inline)) -> float {
        if constexpr (KV::kScaled)
            return ldg<float>(p.q_scale + ((int64_t)x.b * p.R * p.Hq + (int64_t)x.h * p.G),
                              (uint32_t)col.qoff * 4u);
        else
            return 1.f;
    };
    State<D, 1> st;
    typename KV::Q q;
    int nv_cur;
    locate(p, cur, nv_cur);
    load_q_direct<KV>(p, cur, col, ln, q);
    float qs = q_scale_at(cur);
    st.reset();
    __syncthreads();   // the first tile is in LDS
    Fairness fair(by_desc ? sload(p.map, 2) : 1 << 30);
    if (by_desc) fair.start();

    while (true) {
        Pos n;
        const bool more = advance_ahead(d_end, cur, pre, n);
        int nv_n;
        locate(p, pick(more, n, cur), nv_n);
        if (by_desc) fair.tile();
        attend_shared<KV, D>(p, sm, q, qs, nv_cur, col.lag, st, ln);
        __syncthreads();   // done with the tile in LDS

        if (!more || n.d != cur.d) {
            close_descriptor<D, FU>(p, st, sm.last, by_desc ? (int64_t)cur.d : slot_base, cur.b,
                                    cur.h, ln, 64 * NCB);
            if (!more) return;
            pre = read_ahead(src, d_end, n);
            load_q_direct<KV>(p, n, col, ln, q);
            qs = q_scale_at(n);
            st.reset();
        }
        __syncthreads();   // tile t + 1 is in LDS
        cur = n;
        nv_cur = nv_n;
    }
}

// Three workgroups per CU (12 waves) keep enough KV loads in flight; the
// one-block kernel is written to fit the 168 registers per lane that allows.
// More column blocks hold more accumulators and run at two per CU.
template <int NCB>
constexpr int kDecodeWavesPerEu = NCB == 1 ? 3 : 2;

template <class KV, int D, int GR, int NCB, bool MR, bool FU>
__global__ void __launch_bounds__(kDecodeThreads)
__attribute__((amdgpu_waves_per_eu(kDecodeWavesPerEu<NCB>)))
decode_kernel(DecodeParams p) {
    __shared__ MergeLds<D, GR, NCB, KV::kQRowBytes / 4> sm;
    __shared__ KRows<KV::kQRowBytes, KV::kKRows> kr;
    if constexpr (FU) clear_empty_segments<D>(p, kDecodeThreads);
    const MapLayout lay(p.B, p.Hkv, p.P);
    const int32_t *bin_off = p.map + lay.bin_off;
    const int d0 = uniform(bin_off[blockIdx.x]), d1 = uniform(bin_off[blockIdx.x + 1]);
    if (d0 >= d1) return;
    const MapSource src{p.map + lay.desc, p.map + lay.lens};
    drain<KV, D, GR, NCB, MR, FU>(p, sm, k_rows_of(kr), src, src.read(d0), d1, 0, true);
}

// The static ablation keeps the compiler's register allocation (two
// workgroups per CU at D = 128): its grid of many short workgroups ran
// 1-2% faster that way than at the dynamic kernel's three per CU.
template <class KV, int D, int GR, int NCB, bool MR>
__global__ void __launch_bounds__(kDecodeThreads)
static_decode_kernel(DecodeParams p) {
    __shared__ MergeLds<D, GR, NCB, KV::kQRowBytes / 4> sm;
    __shared__ KRows<KV::kQRowBytes, KV::kKRows> kr;
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
        const int RG = rows_per_req<MR>(p) * p.G;
        if ((int)threadIdx.x < RG) p.part_lse[slot * RG + threadIdx.x] = kNegInf;
        return;
    }
    // The same drain as the dynamic kernel, over one range and no map: with
    // d_end = 1 and the range numbered 0 it never reads a descriptor.
    drain<KV, D, GR, NCB, MR, false>(p, sm, k_rows_of(kr), MapSource{nullptr, nullptr},
                                     Pos{0, b, h, (int)t0, (int)t1, L}, 1, slot, false);
}

// Shared-tile kernels (2 .. 4 column blocks): NCB compute waves per
// workgroup, plus a staging wave when SW, sized for three waves per SIMD;
// the bf16 instance with two column blocks and no staging wave needs 190
// registers (hipcc -O3 for gfx950) and runs at two.
template <class KV, int D, int NCB, int SW>
constexpr int shared_waves_per_eu() {
    return (!KV::kScaled && D == 128 && NCB == 2 && SW == 0) ? 2 : 3;
}

template <class KV, int D, int NCB, int SW, bool FU>
__global__ void __launch_bounds__(64 * (NCB + SW))
__attribute__((amdgpu_waves_per_eu(shared_waves_per_eu<KV, D, NCB, SW>())))
decode_shared_kernel(DecodeParams p) {
    __shared__ SharedLds<KV, D> sm;
    if constexpr (FU) clear_empty_segments<D>(p, 64 * (NCB + SW));
    const MapLayout lay(p.B, p.Hkv, p.P);
    const int32_t *bin_off = p.map + lay.bin_off;
    const int d0 = uniform(bin_off[blockIdx.x]), d1 = uniform(bin_off[blockIdx.x + 1]);
    if (d0 >= d1) return;
    const MapSource src{p.map + lay.desc, p.map + lay.lens};
    if constexpr (SW)
        drain_shared_staged<KV, D, NCB, FU>(p, sm, src, src.read(d0), d1, 0, true);
    else
        drain_shared<KV, D, NCB, FU>(p, sm, src, src.read(d0), d1, 0, true);
}

template <class KV, int D, int NCB, int SW>
__global__ void __launch_bounds__(64 * (NCB + SW)) static_decode_shared_kernel(DecodeParams p) {
    __shared__ SharedLds<KV, D> sm;
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
        const int RG = p.R * p.G;
        for (int i = threadIdx.x; i < RG; i += 64 * (NCB + SW))
            p.part_lse[slot * RG + i] = kNegInf;
        return;
    }
    const Pos range{0, b, h, (int)t0, (int)t1, L};
    if constexpr (SW)
        drain_shared_staged<KV, D, NCB, false>(p, sm, MapSource{nullptr, nullptr}, range, 1, slot,
                                               false);
    else
        drain_shared<KV, D, NCB, false>(p, sm, MapSource{nullptr, nullptr}, range, 1, slot, false);
}

// Column blocks of a workgroup: ceil(R G / 16), 1 .. 4.
int column_blocks(int rows) { return (rows + 15) / 16; }

// Whether the shared-tile workgroup for NCB column blocks has a staging
// wave (three column blocks at D = 128).  Each workgroup keeps one tile in
// flight, so the bytes in flight per CU grow with the workgroups it holds.
//   * bf16: three waves would stage 11 chunks (44 registers) per thread,
//     beyond the 168 registers of three waves per SIMD (a spill waits for
//     every load each tile).  A fourth wave holds the 32 chunks per lane
//     instead, next to no accumulators: three workgroups per CU.
//   * fp8: without staging registers the compute waves fit 128 registers,
//     four waves per SIMD, so a CU holds four 4-wave workgroups where it
//     held three 3-wave ones (draft verification, 6 rows of 8 heads:
//     decode 430 -> 364 us).
template <class KV, int D>
constexpr int staging_wave(int ncb) {
    return (ncb == 3 && D == 128) ? 1 : 0;
}

// Workgroups of three waves are held below what their registers allow, by
// padding their LDS.  At three waves per SIMD the registers admit four per
// CU (12 waves), but the dispatcher does not always find SIMDs with room for
// every wave of the fourth: in a launch sized for four per CU some
// workgroups then start only when another ends, and the launch takes up to
// 1.5 times as long.  k = (4 occ - 3) / 3 workgroups leave room for any
// placement of one more workgroup's waves: three at three waves per SIMD,
// four at four.  Computed once per instance from its register count.
//
// The bf16 staging-wave workgroup is held to two per CU, below the three
// its registers admit: with 6 rows of 8 heads, decode + combine ran 1-2%
// faster at two (one process, the same buffers: 311.1 vs 318.4 us and
// 308.0 vs 312.4 us on two boxes), with fewer partials to combine.
constexpr int kLdsPerCu = 160 * 1024;

template <class KV, int D, int NCB, int SW, bool FU>
unsigned shared_lds_pad() {
    constexpr bool staged_bf16 = SW != 0 && !KV::kScaled;
    if constexpr (NCB + SW != 3 && !staged_bf16) {
        return 0u;
    } else {
        static const unsigned pad = [] {
            int k = 2;
            if constexpr (!staged_bf16) {
                hipFuncAttributes a{};
                if (hipFuncGetAttributes(
                        &a, (const void *)decode_shared_kernel<KV, D, NCB, SW, FU>) != hipSuccess)
                    return 0u;
                const int regs = (max(a.numRegs, 1) + 7) / 8 * 8;   // allocation granule
                const int occ = min(8, 512 / regs);                  // waves per SIMD
                k = max(1, (4 * occ - 3) / 3);
            }
            const int want = kLdsPerCu / k - (int)sizeof(SharedLds<KV, D>);
            return want > 0 ? (unsigned)want & ~1023u : 0u;
        }();
        return pad;
    }
}

template <class KV, int D, int NCB>
hipError_t launch_shared(const DecodeParams &p, hipStream_t stream, bool dynamic, int grid) {
    constexpr int SW = staging_wave<KV, D>(NCB);
    if (dynamic && p.out)
        hipLaunchKernelGGL((decode_shared_kernel<KV, D, NCB, SW, true>), dim3(grid),
                           dim3(64 * (NCB + SW)), (shared_lds_pad<KV, D, NCB, SW, true>()),
                           stream, p);
    else if (dynamic)
        hipLaunchKernelGGL((decode_shared_kernel<KV, D, NCB, SW, false>), dim3(grid),
                           dim3(64 * (NCB + SW)), (shared_lds_pad<KV, D, NCB, SW, false>()),
                           stream, p);
    else
        hipLaunchKernelGGL((static_decode_shared_kernel<KV, D, NCB, SW>), dim3(grid),
                           dim3(64 * (NCB + SW)), 0, stream, p);
    return hipGetLastError();
}

// The bf16 per-wave kernel is held to two workgroups per CU by padding its
// LDS, below the three its registers admit: decode + combine ran 0.7%
// faster at two on the mixed batch and 0.4% on heavy-tail, on two boxes
// (one process, the same buffers).  The fp8 kernel, whose tiles are half
// the bytes, keeps three (at two it measured 0.4% slower and 0.4% faster).
// Computed once per instance.
template <class KV, int D, int GR, int NCB, bool MR, bool FU>
unsigned one_row_lds_pad() {
    if constexpr (KV::kScaled) {
        return 0u;
    } else {
        static const unsigned pad = [] {
            hipFuncAttributes a{};
            if (hipFuncGetAttributes(&a, (const void *)decode_kernel<KV, D, GR, NCB, MR, FU>) !=
                hipSuccess)
                return 0u;
            const int want = kLdsPerCu / 2 - (int)a.sharedSizeBytes;
            return want > 0 ? (unsigned)want & ~1023u : 0u;
        }();
        return pad;
    }
}

template <class KV, int D, int GR, int NCB, bool MR>
hipError_t launch_one(const DecodeParams &p, hipStream_t stream, bool dynamic, int grid) {
    if (dynamic && p.out)
        hipLaunchKernelGGL((decode_kernel<KV, D, GR, NCB, MR, true>), dim3(grid),
                           dim3(kDecodeThreads), (one_row_lds_pad<KV, D, GR, NCB, MR, true>()),
                           stream, p);
    else if (dynamic)
        hipLaunchKernelGGL((decode_kernel<KV, D, GR, NCB, MR, false>), dim3(grid),
                           dim3(kDecodeThreads), (one_row_lds_pad<KV, D, GR, NCB, MR, false>()),
                           stream, p);
    else
        hipLaunchKernelGGL((static_decode_kernel<KV, D, GR, NCB, MR>), dim3(grid),
                           dim3(kDecodeThreads), 0, stream, p);
    return hipGetLastError();
}

// The instance for R G query rows: one 16-column block (8-row merge buffer
// up to 8 rows), specialised for R = 1, or the shared-tile path for 2 .. 4
// blocks.
template <template <int> class KV, int D>
hipError_t launch_for(const DecodeParams &p, hipStream_t stream, bool dynamic, int grid) {
    const int rows = p.R * p.G;
    switch (column_blocks(rows)) {
    case 1:
        if (p.R == 1)
            return rows <= 8 ? launch_one<KV<D>, D, 8, 1, false>(p, stream, dynamic, grid)
                             : launch_one<KV<D>, D, 16, 1, false>(p, stream, dynamic, grid);
        return rows <= 8 ? launch_one<KV<D>, D, 8, 1, true>(p, stream, dynamic, grid)
                         : launch_one<KV<D>, D, 16, 1, true>(p, stream, dynamic, grid);
    case 2: return launch_shared<KV<D>, D, 2>(p, stream, dynamic, grid);
    case 3: return launch_shared<KV<D>, D, 3>(p, stream, dynamic, grid);
    default: return launch_shared<KV<D>, D, 4>(p, stream, dynamic, grid);
    }
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

// The dynamic kernel launch_for picks for `rows` rows with R = 1 when
// rows <= 16 (the resident count does not depend on R otherwise), with the
// combine fused (FU) or not.
template <template <int> class KV, int D, bool FU>
const void *decode_fn(int rows, int &threads, unsigned &lds_pad) {
    constexpr int SW2 = staging_wave<KV<D>, D>(2), SW3 = staging_wave<KV<D>, D>(3),
                  SW4 = staging_wave<KV<D>, D>(4);
    const int ncb = column_blocks(rows);
    threads = ncb == 1 ? kDecodeThreads : 64 * (ncb + staging_wave<KV<D>, D>(ncb));
    lds_pad = ncb == 3 ? shared_lds_pad<KV<D>, D, 3, SW3, FU>() : 0u;
    switch (ncb) {
    case 1:
        lds_pad = rows <= 8 ? one_row_lds_pad<KV<D>, D, 8, 1, false, FU>()
                            : one_row_lds_pad<KV<D>, D, 16, 1, false, FU>();
        return rows <= 8 ? (const void *)decode_kernel<KV<D>, D, 8, 1, false, FU>
                         : (const void *)decode_kernel<KV<D>, D, 16, 1, false, FU>;
    case 2: return (const void *)decode_shared_kernel<KV<D>, D, 2, SW2, FU>;
    case 3: return (const void *)decode_shared_kernel<KV<D>, D, 3, SW3, FU>;
    default: return (const void *)decode_shared_kernel<KV<D>, D, 4, SW4, FU>;
    }
}

template <bool FU>
int32_t resident_per_cu(int32_t head_dim, int32_t kv_dtype, int32_t rows) {
    int n = 0;
    int threads = 0;
    unsigned pad = 0;
    const void *fn = kv_dtype == HPCATTN_KV_BF16
                         ? (head_dim == 128 ? decode_fn<Bf16, 128, FU>(rows, threads, pad)
                                            : decode_fn<Bf16, 64, FU>(rows, threads, pad))
                         : (head_dim == 128 ? decode_fn<Fp8, 128, FU>(rows, threads, pad)
                                            : decode_fn<Fp8, 64, FU>(rows, threads, pad));
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, pad) != hipSuccess)
        return 0;
    return n;
}

}  // namespace

int32_t decode_resident_per_cu(int32_t head_dim, int32_t kv_dtype, int32_t rows) {
    return resident_per_cu<false>(head_dim, kv_dtype, rows);
}

bool fused_keeps_residency(int32_t head_dim, int32_t kv_dtype, int32_t rows) {
    // One answer per instance pair (dtype, head_dim, column blocks, and for
    // one block whether rows <= 8), looked up once: 0 unknown, 1 no, 2 yes.
    static std::atomic<int> known[2][2][5];
    const int ncb = column_blocks(rows);
    std::atomic<int> &k = known[kv_dtype == HPCATTN_KV_BF16 ? 0 : 1][head_dim == 128 ? 1 : 0]
                               [ncb == 1 ? (rows <= 8 ? 0 : 1) : ncb];
    int v = k.load(std::memory_order_relaxed);
    if (v == 0) {
        const int32_t n = resident_per_cu<false>(head_dim, kv_dtype, rows);
        v = n > 0 && resident_per_cu<true>(head_dim, kv_dtype, rows) == n ? 2 : 1;
        k.store(v, std::memory_order_relaxed);
    }
    return v == 2;
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
