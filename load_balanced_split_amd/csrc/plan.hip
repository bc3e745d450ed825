// The assign step: build the task map on the device from device-side lengths.
//
// "HPC-Ops x SGLang", section "Scheduling around live KV work": each sequence
// is cut into uniform 64-token tiles, the tile counts are summed over all
// heads and requests, the total divided by the number of persistent
// workgroups sets the per-bin budget, and each bin is filled to its budget
// before spilling into the next, with a minimum-work floor.  "Hy3 preview
// full-stack inference optimization", section 2.1.1: greedy bin packing over
// a global tile total, the map built once before each step.
//
// The integer reading used throughout: segments s = b * H_kv + h of
// n_b = ceil(L_b / 64) tiles, in that order; P_eff = min(P, max(1, T / m))
// bins, bin i owning global tiles [i q + min(i, r), (i + 1) q + min(i + 1, r))
// with T = q P_eff + r.  A descriptor is one (bin, segment) intersection.
//
// One workgroup of 1024 threads.  Segment s starts at global tile
// H_kv * cum(b) + h * n_b, where cum is the exclusive scan of n over
// requests, so only the request scan needs storage (LDS); chunk counts per
// segment come from the closed-form bin of a tile, and their scan gives the
// descriptor numbering, which is also the global tile order.
#include "common.h"

namespace hpcattn {
namespace {

constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kWaveChunks = 32;   // segments with more descriptors are written by a wave
constexpr int kWideList = 64;     // such segments spread over all waves; more: their own wave

struct Bins {
    int64_t T, P_eff, q, r;
    // First global tile of bin i (bins past P_eff are empty at T).
    __device__ int64_t start(int64_t i) const {
        return i <= P_eff ? i * q + (i < r ? i : r) : T;
    }
    // Bin that owns global tile x, 0 <= x < T (then q >= 1).  T fits in 31
    // bits (a larger total is refused), so 32-bit division suffices.
    __device__ int64_t of(int64_t x) const {
        const int64_t big = r * (q + 1);
        return x < big ? (uint32_t)x / (uint32_t)(q + 1)
                       : r + (uint32_t)(x - big) / (uint32_t)q;
    }
};

// Lane l's value of v, l uniform across the wave (read into scalar registers).
__device__ inline int64_t lane_value(int64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), l);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ int64_t wave_inclusive_scan(int64_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t n = __shfl_up(v, o, 64);
        if (lane >= o) v += n;
    }
    return v;
}

// Exclusive scan of one value per thread over the workgroup, in thread
// order; *total receives the sum.  Contains barriers: call from all threads.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t *total, int64_t *s_wave) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t inc = wave_inclusive_scan(v);
    if (lane == 63) s_wave[w] = inc;
    __syncthreads();
    int64_t base = 0, all = 0;
    for (int i = 0; i < kPlanWaves; ++i) {
        const int64_t x = s_wave[i];
        base += i < w ? x : 0;
        all += x;
    }
    __syncthreads();
    *total = all;
    return base + inc - v;
}

__device__ inline int64_t tiles_of(int32_t len) {
    return len > 0 ? ((int64_t)len + kTile - 1) / kTile : 0;
}

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(const int32_t *__restrict__ seq_lens, int32_t B, int32_t Hkv, int32_t P,
            int32_t m, int32_t *__restrict__ map) {
    __shared__ int32_t s_cum[HPCATTN_MAX_BATCH + 1];   // tiles before request b; [B] = all
    __shared__ int64_t s_wave[kPlanWaves];
    __shared__ int64_t s_wide[kWideList][7];   // b, h, st, en, j0, c, first descriptor
    __shared__ int32_t s_err, s_nwide;

    const MapLayout lay(B, Hkv, P);
    int32_t *lens_out = map + lay.lens;
    int32_t *bin_off = map + lay.bin_off;
    int32_t *seg_off = map + lay.seg_off;
    int32_t *desc = map + lay.desc;
    const int tid = threadIdx.x;
    const int64_t S = (int64_t)B * Hkv;
    const int64_t Dmax = S + P - 1;

    if (tid == 0) {
        s_err = 0;
        s_nwide = 0;
    }
    __syncthreads();

    // Phase A: tiles per request and their exclusive scan over requests.
    const int per_b = (B + kPlanThreads - 1) / kPlanThreads;
    const int b0 = tid * per_b, b1 = min(B, b0 + per_b);
    int64_t local = 0;
    for (int b = b0; b < b1; ++b) {
        const int32_t L = seq_lens[b];
        if (L < 0) s_err = HPCATTN_MAPERR_NEG_LEN;
        lens_out[b] = L > 0 ? L : 0;
        local += tiles_of(L);
    }
    int64_t n_total;
    int64_t run = block_exclusive_scan(local, &n_total, s_wave);
    for (int b = b0; b < b1; ++b) {
        s_cum[b] = (int32_t)run;
        run += tiles_of(seq_lens[b]);
    }
    if (tid == 0) s_cum[B] = (int32_t)n_total;   // (meaningless on overflow, then unused)
    bool overflow = n_total * Hkv > (int64_t)INT32_MAX;
    if (overflow && tid == 0) s_err = HPCATTN_MAPERR_OVERFLOW;
    __syncthreads();

    // Phase B: the budget with the minimum-work floor.  On overflow the map
    // describes no work at all.
    Bins bins;
    bins.T = overflow ? 0 : n_total * Hkv;
    bins.P_eff = bins.T / m;
    if (bins.P_eff < 1) bins.P_eff = 1;
    if (bins.P_eff > P) bins.P_eff = P;
    bins.q = bins.T / bins.P_eff;
    bins.r = bins.T % bins.P_eff;

    // Phase C: chunk count of every segment and their exclusive scan, over
    // per_s consecutive segments per thread.
    const int64_t per_s = (S + kPlanThreads - 1) / kPlanThreads;
    const int64_t s0 = tid * per_s, s1 = min(S, s0 + per_s);
    // Segment s: request b, head h, global tiles [st, en), first bin j0 and
    // chunk count c.  s < 2^31 (larger sizes are refused).
    struct Seg {
        int b, h;
        int64_t st, en, j0, c;
    };
    auto seg = [&](int64_t s) -> Seg {
        Seg g;
        g.b = (int)((uint32_t)s / (uint32_t)Hkv);
        g.h = (int)((uint32_t)s - (uint32_t)g.b * (uint32_t)Hkv);
        const int64_t n = s_cum[g.b + 1] - s_cum[g.b];
        g.st = (int64_t)Hkv * s_cum[g.b] + g.h * n;
        g.en = g.st + n;
        g.j0 = n ? bins.of(g.st) : 0;
        g.c = n ? bins.of(g.en - 1) - g.j0 + 1 : 0;
        return g;
    };
    local = 0;
    if (!overflow)
        for (int64_t s = s0; s < s1; ++s) local += seg(s).c;
    int64_t num_desc;
    run = block_exclusive_scan(local, &num_desc, s_wave);

    // Phase D: per-segment offsets and descriptors.  Each descriptor is the
    // intersection of segment s with one bin j; a bin's first descriptor also
    // sets its bin offset.  A thread writes the descriptors of its segment of
    // the round.  A segment of more than kWaveChunks (a long request spans
    // hundreds of bins) is written by a whole wave, a lane per descriptor:
    // the first kWideList such segments are listed in LDS and spread over all
    // the waves afterwards (a few long requests would otherwise all fall to
    // the waves that own them); any further ones by the wave that owns them,
    // one at a time.
    auto put = [&](const Seg &g, int64_t i, int64_t d) {   // chunk i of g is descriptor d
        const int64_t j = g.j0 + i, bs = bins.start(j), be = bins.start(j + 1);
        const int64_t lo = bs > g.st ? bs : g.st, hi = be < g.en ? be : g.en;
        int32_t *d4 = desc + 4 * d;
        d4[0] = g.b;
        d4[1] = g.h;
        d4[2] = (int32_t)(lo - g.st);
        d4[3] = (int32_t)(hi - g.st);
        if (i > 0 || g.st == bs) bin_off[j] = (int32_t)d;
    };
    const int lane = tid & 63;
    for (int64_t round = 0; round < per_s; ++round) {   // the same count in every wave
        const int64_t s = s0 + round;
        Seg g{0, 0, 0, 0, 0, 0};
        if (s < s1) {
            seg_off[s] = (int32_t)run;
            if (!overflow) g = seg(s);
        }
        const bool wide = g.c > kWaveChunks;
        if (!wide)
            for (int64_t i = 0; i < g.c; ++i) put(g, i, run + i);
        bool listed = false;
        if (wide) {
            const int k = atomicAdd(&s_nwide, 1);
            if (k < kWideList) {
                const int64_t e[7] = {g.b, g.h, g.st, g.en, g.j0, g.c, run};
#pragma unroll
                for (int f = 0; f < 7; ++f) s_wide[k][f] = e[f];
                listed = true;
            }
        }
        for (uint64_t longs = __ballot(wide && !listed); longs; longs &= longs - 1) {
            const int l = __ffsll((unsigned long long)longs) - 1;   // wave-uniform
            Seg w;
            w.b = (int)lane_value(g.b, l);
            w.h = (int)lane_value(g.h, l);
            w.st = lane_value(g.st, l);
            w.en = lane_value(g.en, l);
            w.j0 = lane_value(g.j0, l);
            w.c = lane_value(g.c, l);
            const int64_t first = lane_value(run, l);
            for (int64_t k = lane; k < w.c; k += 64) put(w, k, first + k);
        }
        run += g.c;
    }
    if (tid == 0) seg_off[S] = (int32_t)num_desc;
    __syncthreads();
    for (int i = tid >> 6; i < min(s_nwide, kWideList); i += kPlanWaves) {   // wave-uniform i
        const Seg w{(int)s_wide[i][0], (int)s_wide[i][1], s_wide[i][2],
                    s_wide[i][3],      s_wide[i][4],      s_wide[i][5]};
        for (int64_t k = lane; k < w.c; k += 64) put(w, k, s_wide[i][6] + k);
    }

    // Phase E: bins that own no tile start at num_desc.
    for (int64_t j = tid; j <= P; j += kPlanThreads)
        if (bins.start(j) >= bins.T) bin_off[j] = (int32_t)num_desc;

    // Phase F: unused descriptor slots are zero.
    for (int64_t w = 4 * num_desc + tid; w < 4 * Dmax; w += kPlanThreads) desc[w] = 0;

    __syncthreads();
    if (tid == 0) {
        map[0] = (int32_t)bins.T;
        map[1] = (int32_t)bins.P_eff;
        map[2] = (int32_t)bins.q;
        map[3] = (int32_t)bins.r;
        map[4] = (int32_t)num_desc;
        map[5] = B;
        map[6] = Hkv;
        map[7] = s_err;
    }
}

}  // namespace

hipError_t launch_plan(const int32_t *seq_lens, int32_t B, int32_t Hkv, int32_t P,
                       int32_t m, int32_t *map, hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, B,
                       Hkv, P, m, map);
    return hipGetLastError();
}

}  // namespace hpcattn
