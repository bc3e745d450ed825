/*
 * oracle.c -- plain, slow, fp64 CPU reference for load-balanced split-KV
 * decode attention over a paged GQA KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library: the task-map layout below is written from its textual
 * specification (the C-ABI header documents the same layout), not included.
 *
 * Sources (the pages this method is described on):
 *   [HPC-Ops] "HPC-Ops x SGLang: Tencent Hunyuan open-sources high-performance
 *             Attention, Router GEMM and MoE operators", sections
 *             "Attention: load balancing for variable-length decode" and
 *             "Scheduling around live KV work", and "Fused attention prologue".
 *   [Hy3]     "Hy3 preview full-stack inference optimization", section 2.1.1
 *             "Attention dynamic scheduling", and section 2.5 (MTP: the
 *             target model verifies the draft tokens of a step).
 *   [LowLat]  "SGLang Low-Latency Mode: Kernels and Runtime", section 1: a
 *             verify step runs one forward over six rows per request, the
 *             confirmed token and five drafts.
 *
 * Parity pins (all in the CPU test suite): a numpy brute-force softmax on tiny
 * inputs, torch float64 scaled-dot-product attention as a library routine,
 * closed forms, the split/merge identity, a per-tile greedy bin fill, and the
 * OCP E4M3FN code table.  No function here is "parity unpinned".
 *
 * Build:  gcc -O2 -std=c11 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One tile is 64 tokens, and one KV page holds 64 tokens
 * ([HPC-Ops] "Scheduling around live KV work": sequences are cut into
 * uniform 64-token tiles; the serving setup uses page size 64). */
#define ORC_TILE 64

typedef struct {
    int32_t batch;        /* B                                           */
    int32_t num_q_heads;  /* H_q                                         */
    int32_t num_kv_heads; /* H_kv; H_q is a multiple of it               */
    int32_t head_dim;     /* D                                           */
    int32_t max_pages;    /* columns of page_table                       */
    int32_t num_pages;    /* pages in each KV pool                       */
    int32_t kv_fp8;       /* 0: bf16 q/k/v; 1: fp8 e4m3 bytes + scales   */
    int32_t q_rows;       /* R >= 1 query rows per request (1 + drafts)  */
    double sm_scale;      /* softmax scale applied to q.k                */
} orc_dims;

/* ------------------------------------------------------------------ */
/* Element decoders, written from the format definitions.              */
/* ------------------------------------------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE binary32.  Exact in fp64. */
double orc_bf16_value(int32_t bits)
{
    uint32_t w = ((uint32_t)bits & 0xFFFFu) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* OCP 8-bit E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits.  Exponent field 0 encodes subnormals m/8 * 2^-6.  There are no
 * infinities; S.1111.111 is NaN, so the largest finite value is
 * 1.75 * 2^8 = 448.  ([HPC-Ops] "Fused attention prologue" and the serving
 * setup use an fp8_e4m3 KV cache; the value is code * scale.) */
double orc_e4m3_value(int32_t code)
{
    uint32_t c = (uint32_t)code & 0xFFu;
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Query rows per request: R = 1 for plain decode, 1 + k when a step     */
/* verifies k draft tokens in one forward ([Hy3] 2.5; [LowLat] 1).      */
static int rows_of(const orc_dims *dm)
{
    return dm->q_rows > 1 ? dm->q_rows : 1;
}

/* ------------------------------------------------------------------ */
/* Paged KV access.                                                     */
/*   q          [B, R, H_q, D]         bf16 bits or e4m3 bytes         */
/*   q_scale    [B, R, H_q]            fp32 (fp8 only)                 */
/*   k/v pools  [num_pages, H_kv, 64, D]                               */
/*   k/v scale  [num_pages, H_kv, 64]  fp32 (fp8 only)                 */
/*   page_table [B, max_pages]         int32; token t of request b is  */
/*              slot t mod 64 of page page_table[b][t / 64].           */
/* ------------------------------------------------------------------ */

static double load_q(const orc_dims *dm, const void *q, const float *q_scale,
                     int b, int r, int j, int d)
{
    int64_t row = ((int64_t)b * rows_of(dm) + r) * dm->num_q_heads + j;
    int64_t idx = row * dm->head_dim + d;
    if (dm->kv_fp8)
        return orc_e4m3_value(((const uint8_t *)q)[idx]) * (double)q_scale[row];
    return orc_bf16_value(((const uint16_t *)q)[idx]);
}

static double load_kv(const orc_dims *dm, const void *pool, const float *scale,
                      int64_t page, int h, int slot, int d)
{
    int64_t row = (page * dm->num_kv_heads + h) * ORC_TILE + slot;
    int64_t idx = row * dm->head_dim + d;
    if (dm->kv_fp8)
        return orc_e4m3_value(((const uint8_t *)pool)[idx]) * (double)scale[row];
    return orc_bf16_value(((const uint16_t *)pool)[idx]);
}

/* ------------------------------------------------------------------ */
/* Attention of the query rows of one (request, KV head) over a token   */
/* range.                                                               */
/*                                                                      */
/* For request b, query row r and query head j (KV head h = j / G,      */
/* G = H_q / H_kv):                                                     */
/*   s_t = sm_scale * sum_d q_d k_{t,d}                                 */
/*   M   = max_t s_t,  l = sum_t exp(s_t - M)                           */
/*   o   = sum_t exp(s_t - M) v_t / l,   lse = M + ln l                 */
/* over tokens t in [tok0, min(tok1, len - (R - 1 - r))), len = L_b.    */
/* With R = 1 the new token attends over the whole cached KV of its     */
/* request, with no other mask ([HPC-Ops] "Attention: load balancing    */
/* for variable-length decode").  With R > 1 the R rows are the last R  */
/* tokens of the request (the cache already holds all of them), row r   */
/* at position len - R + r, and each sees the tokens up to and          */
/* including its own: a causal mask among the drafts ([Hy3] 2.5 and     */
/* [LowLat] 1 verify drafts in one forward; the pages give no mask, and */
/* the causal one is the plain reading of verifying a token sequence).  */
/* An empty range gives o = 0, lse = -inf.                              */
/* Writes o [R * G, D] and lse [R * G], row r * G + g for head h G + g. */
/* ------------------------------------------------------------------ */
int orc_attend_range(const orc_dims *dm, const void *q, const float *q_scale,
                     const void *k_pages, const void *v_pages,
                     const float *k_scale, const float *v_scale,
                     const int32_t *page_table, int32_t b, int32_t h,
                     int32_t tok0, int32_t tok1, int32_t len,
                     double *o /* [R * G, D] */, double *lse /* [R * G] */)
{
    const int D = dm->head_dim;
    const int G = dm->num_q_heads / dm->num_kv_heads;
    const int R = rows_of(dm);
    const int span = tok1 > tok0 ? tok1 - tok0 : 0;
    double *s = (double *)malloc(sizeof(double) * (span > 0 ? span : 1));
    double *qv = (double *)malloc(sizeof(double) * D);
    if (!s || !qv) {
        free(s);
        free(qv);
        return -1;
    }
    for (int c = 0; c < R * G; ++c) {
        int r = c / G, g = c % G;
        int j = h * G + g;
        int end = len - (R - 1 - r);   /* tokens row r may see */
        if (end > tok1)
            end = tok1;
        const int n = end > tok0 ? end - tok0 : 0;
        double *og = o + (int64_t)c * D;
        for (int d = 0; d < D; ++d) {
            qv[d] = load_q(dm, q, q_scale, b, r, j, d);
            og[d] = 0.0;
        }
        if (n == 0) {
            lse[c] = -INFINITY;
            continue;
        }
        double M = -INFINITY;
        for (int i = 0; i < n; ++i) {
            int t = tok0 + i;
            int64_t page = page_table[(int64_t)b * dm->max_pages + t / ORC_TILE];
            double acc = 0.0;
            for (int d = 0; d < D; ++d)
                acc += qv[d] * load_kv(dm, k_pages, k_scale, page, h, t % ORC_TILE, d);
            s[i] = dm->sm_scale * acc;
            if (s[i] > M)
                M = s[i];
        }
        double l = 0.0;
        for (int i = 0; i < n; ++i) {
            int t = tok0 + i;
            int64_t page = page_table[(int64_t)b * dm->max_pages + t / ORC_TILE];
            double p = exp(s[i] - M);
            l += p;
            for (int d = 0; d < D; ++d)
                og[d] += p * load_kv(dm, v_pages, v_scale, page, h, t % ORC_TILE, d);
        }
        for (int d = 0; d < D; ++d)
            og[d] /= l;
        lse[c] = M + log(l);
    }
    free(s);
    free(qv);
    return 0;
}

/* Full decode attention: every request over its whole live KV.
 * pairs: NULL for all (b, h) pairs, else n_pairs (b, h) int32 pairs; only
 * those rows of out/out_lse are written.  out [B, R, H_q, D],
 * out_lse [B, R, H_q].  One OpenMP task per (request, KV head), all R G
 * query rows together. */
int orc_attention(const orc_dims *dm, const void *q, const float *q_scale,
                  const void *k_pages, const void *v_pages,
                  const float *k_scale, const float *v_scale,
                  const int32_t *page_table, const int32_t *seq_lens,
                  const int32_t *pairs, int32_t n_pairs,
                  double *out, double *out_lse)
{
    const int H_kv = dm->num_kv_heads;
    const int G = dm->num_q_heads / H_kv;
    const int D = dm->head_dim;
    const int R = rows_of(dm);
    const int64_t total = pairs ? n_pairs : (int64_t)dm->batch * H_kv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t i = 0; i < total; ++i) {
        int b = pairs ? pairs[2 * i] : (int)(i / H_kv);
        int h = pairs ? pairs[2 * i + 1] : (int)(i % H_kv);
        double *o = (double *)malloc(sizeof(double) * (size_t)R * G * D);
        double *l = (double *)malloc(sizeof(double) * (size_t)R * G);
        if (!o || !l) {
            free(o);
            free(l);
            err |= 1;
            continue;
        }
        err |= orc_attend_range(dm, q, q_scale, k_pages, v_pages, k_scale, v_scale,
                                page_table, b, h, 0, seq_lens[b], seq_lens[b], o, l);
        for (int c = 0; c < R * G; ++c) {
            int64_t row = ((int64_t)b * R + c / G) * dm->num_q_heads + (int64_t)h * G + c % G;
            memcpy(out + row * D, o + (int64_t)c * D, sizeof(double) * D);
            out_lse[row] = l[c];
        }
        free(o);
        free(l);
    }
    return err ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* Log-sum-exp merge of n partial results, each normalised with its own */
/* lse, into the result under the global softmax ([HPC-Ops] "Scheduling */
/* around live KV work": the combine merges the partials under the      */
/* correct global softmax normalisation).                               */
/*   M = max_i lse_i,  w_i = exp(lse_i - M)                             */
/*   out = sum_i w_i o_i / sum_i w_i,  out_lse = M + ln sum_i w_i       */
/* Partials with lse = -inf carry no weight; if all are -inf (or n = 0) */
/* out = 0 and out_lse = -inf.                                          */
/* ------------------------------------------------------------------ */
void orc_lse_merge(int32_t n, int32_t width, const double *lse, const double *o,
                   double *out, double *out_lse)
{
    double M = -INFINITY;
    for (int i = 0; i < n; ++i)
        if (lse[i] > M)
            M = lse[i];
    for (int d = 0; d < width; ++d)
        out[d] = 0.0;
    if (M == -INFINITY) {
        *out_lse = -INFINITY;
        return;
    }
    double wsum = 0.0;
    for (int i = 0; i < n; ++i) {
        if (lse[i] == -INFINITY)
            continue;
        double w = exp(lse[i] - M);
        wsum += w;
        for (int d = 0; d < width; ++d)
            out[d] += w * o[(int64_t)i * width + d];
    }
    for (int d = 0; d < width; ++d)
        out[d] /= wsum;
    *out_lse = M + log(wsum);
}

/* ------------------------------------------------------------------ */
/* Task map: which tiles each persistent workgroup owns.                */
/*                                                                      */
/* [HPC-Ops] "Scheduling around live KV work" and [Hy3] 2.1.1: cut each */
/* sequence into uniform 64-token tiles, sum the tile counts across all */
/* heads and requests, divide the total by the number of persistent     */
/* workgroups to set a per-workgroup tile budget, fill each bin to the  */
/* budget and spill into the next; a minimum-work floor stops           */
/* over-partitioning when the total is small.                           */
/*                                                                      */
/* Readings where the pages leave a step open:                          */
/*  - tiles are counted per (request, KV head) segment; a partial last  */
/*    tile counts as one tile;                                           */
/*  - segments are ordered s = b * H_kv + h, tiles in order within one; */
/*  - the budget is the integer split T = q * P_eff + r: the first r    */
/*    bins take q + 1 tiles and the rest q;                              */
/*  - the floor: P_eff = min(P, max(1, T / m)) bins are used, the other */
/*    P - P_eff bins are empty;                                          */
/*  - a descriptor is the part of one segment inside one bin, and its   */
/*    index is its partial-result slot.                                 */
/*                                                                      */
/* Layout (int32 words):                                                */
/*   [0..7]   header {T, P_eff, q, r, num_desc, B, H_kv, err}           */
/*   [8..]    seq_lens[B]                                               */
/*            bin_desc_off[P + 1]                                       */
/*            seg_desc_off[B * H_kv + 1]                                */
/*            desc[B * H_kv + P - 1][4] = {b, h, t0, t1}, tiles [t0,t1) */
/* ------------------------------------------------------------------ */

int64_t orc_plan_words(int32_t B, int32_t H_kv, int32_t P)
{
    int64_t segs = (int64_t)B * H_kv;
    return 8 + (int64_t)B + ((int64_t)P + 1) + (segs + 1) + 4 * (segs + P - 1);
}

/* Returns the number of words written, or a negative value on bad input. */
int64_t orc_plan(const int32_t *seq_lens, int32_t B, int32_t H_kv, int32_t P,
                 int32_t m, int32_t *map, int64_t map_words)
{
    if (B < 1 || H_kv < 1 || P < 1 || m < 1 || !seq_lens || !map)
        return -1;
    const int64_t words = orc_plan_words(B, H_kv, P);
    if (map_words < words)
        return -2;
    const int64_t S = (int64_t)B * H_kv;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0)
            return -3;

    int32_t *hdr = map;
    int32_t *lens = hdr + 8;
    int32_t *bin_off = lens + B;
    int32_t *seg_off = bin_off + (P + 1);
    int32_t *desc = seg_off + (S + 1);
    memset(map, 0, sizeof(int32_t) * (size_t)words);

    /* Step 1: tiles per segment and their exclusive prefix scan. */
    int64_t *seg_start = (int64_t *)malloc(sizeof(int64_t) * (size_t)(S + 1));
    if (!seg_start)
        return -4;
    seg_start[0] = 0;
    for (int64_t s = 0; s < S; ++s) {
        int b = (int)(s / H_kv);
        int64_t n_b = ((int64_t)seq_lens[b] + ORC_TILE - 1) / ORC_TILE;
        seg_start[s + 1] = seg_start[s] + n_b;
    }
    const int64_t T = seg_start[S];
    if (T > INT32_MAX) {
        free(seg_start);
        return -5;
    }

    /* Step 2: the budget with the minimum-work floor. */
    int64_t P_eff = T / m;
    if (P_eff < 1)
        P_eff = 1;
    if (P_eff > P)
        P_eff = P;
    const int64_t q = T / P_eff, r = T % P_eff;

    /* Step 3: bin i owns global tiles [bin_start(i), bin_start(i + 1)). */
#define BIN_START(i) ((i) <= P_eff ? (i) * q + ((i) < r ? (i) : r) : T)

    /* Step 4: descriptors = non-empty (bin range) x (segment range)
     * intersections, numbered in increasing global tile order. */
    int64_t nd = 0;
    int64_t s = 0;
    for (int64_t i = 0; i < P; ++i) {
        int64_t lo = BIN_START(i), hi = BIN_START(i + 1);
        bin_off[i] = (int32_t)nd;
        while (s < S && seg_start[s + 1] <= lo)
            ++s;
        for (int64_t u = s; u < S && seg_start[u] < hi; ++u) {
            int64_t a = lo > seg_start[u] ? lo : seg_start[u];
            int64_t z = hi < seg_start[u + 1] ? hi : seg_start[u + 1];
            if (a >= z)
                continue;
            int32_t *d4 = desc + 4 * nd;
            d4[0] = (int32_t)(u / H_kv);
            d4[1] = (int32_t)(u % H_kv);
            d4[2] = (int32_t)(a - seg_start[u]);
            d4[3] = (int32_t)(z - seg_start[u]);
            ++nd;
        }
    }
    bin_off[P] = (int32_t)nd;
#undef BIN_START

    /* Step 5: per-segment CSR over the same numbering. */
    {
        int64_t k = 0;
        for (int64_t u = 0; u < S; ++u) {
            seg_off[u] = (int32_t)k;
            while (k < nd && (int64_t)desc[4 * k] * H_kv + desc[4 * k + 1] == u)
                ++k;
        }
        seg_off[S] = (int32_t)k;
    }

    for (int b = 0; b < B; ++b)
        lens[b] = seq_lens[b];
    hdr[0] = (int32_t)T;
    hdr[1] = (int32_t)P_eff;
    hdr[2] = (int32_t)q;
    hdr[3] = (int32_t)r;
    hdr[4] = (int32_t)nd;
    hdr[5] = B;
    hdr[6] = H_kv;
    hdr[7] = 0;
    free(seg_start);
    return words;
}

/* Per-descriptor partials following a task map: descriptor k covers
 * tokens [64 t0, 64 t1) of segment (b, h), each query row within its own
 * visible length (orc_attend_range).  Writes part_o [num_desc, R G, D] and
 * part_lse [num_desc, R G].  P is the bin count
 * the map was planned with (it fixes the layout offsets).
 * ([HPC-Ops] "Scheduling around live KV work": each workgroup writes a
 * partial output with its log-sum-exp for every descriptor it drains). */
int orc_partials(const orc_dims *dm, const void *q, const float *q_scale,
                 const void *k_pages, const void *v_pages,
                 const float *k_scale, const float *v_scale,
                 const int32_t *page_table, const int32_t *map, int32_t P,
                 double *part_o, double *part_lse)
{
    const int B = map[5], H_kv = map[6];
    const int G = dm->num_q_heads / dm->num_kv_heads;
    const int D = dm->head_dim;
    const int R = rows_of(dm);
    const int64_t nd = map[4];
    const int64_t S = (int64_t)B * H_kv;
    const int32_t *lens = map + 8;
    const int32_t *desc = map + 8 + B + (P + 1) + (S + 1);
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t k = 0; k < nd; ++k) {
        const int32_t *d4 = desc + 4 * k;
        int b = d4[0], h = d4[1];
        int tok0 = d4[2] * ORC_TILE;
        int tok1 = d4[3] * ORC_TILE;
        err |= orc_attend_range(dm, q, q_scale, k_pages, v_pages, k_scale, v_scale,
                                page_table, b, h, tok0, tok1, lens[b],
                                part_o + k * R * G * D, part_lse + k * R * G);
    }
    return err ? -1 : 0;
}

/* Merge the partials of each segment (its descriptors are the contiguous
 * run seg_desc_off[s] .. seg_desc_off[s + 1]), row by row, into
 * out [B, R, H_q, D] and out_lse [B, R, H_q].  P is the bin count the map
 * was planned with. */
int orc_combine(const orc_dims *dm, const int32_t *map, int32_t P,
                const double *part_o, const double *part_lse,
                double *out, double *out_lse)
{
    const int B = map[5], H_kv = map[6];
    const int G = dm->num_q_heads / dm->num_kv_heads;
    const int D = dm->head_dim;
    const int R = rows_of(dm);
    const int64_t S = (int64_t)B * H_kv;
    const int32_t *seg_off = map + 8 + B + (P + 1);
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t s = 0; s < S; ++s) {
        int b = (int)(s / H_kv), h = (int)(s % H_kv);
        int k0 = seg_off[s], k1 = seg_off[s + 1];
        int n = k1 - k0;
        double *lse = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
        double *og = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
        if (!lse || !og) {
            free(lse);
            free(og);
            err |= 1;
            continue;
        }
        for (int c = 0; c < R * G; ++c) {
            for (int i = 0; i < n; ++i) {
                lse[i] = part_lse[(int64_t)(k0 + i) * R * G + c];
                memcpy(og + (int64_t)i * D, part_o + ((int64_t)(k0 + i) * R * G + c) * D,
                       sizeof(double) * D);
            }
            int64_t row = ((int64_t)b * R + c / G) * dm->num_q_heads + (int64_t)h * G + c % G;
            orc_lse_merge(n, D, lse, og, out + row * D, out_lse + row);
        }
        free(lse);
        free(og);
    }
    return err ? -1 : 0;
}

int32_t orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_threads(int32_t n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------ */
/* The attention prologue after the QKV projection ([HPC-Ops] "Fused  */
/* attention prologue"; [Hy3] 2.2.1 "Fused Rope+Norm+[Hadamard]+Quant */
/* +Store KV"): QK-Norm before RoPE, an optional Hadamard rotation of  */
/* Q and K before quantisation ([Hy3] 2.6.1, online rotation), Q      */
/* quantised to fp8 with a per-token per-head scale, K and V quantised */
/* and written straight into the paged cache.                          */
/*                                                                      */
/* Readings where the pages are silent:                                 */
/*  - QK-Norm is RMSNorm over each head's D values with a learned       */
/*    weight per dimension (one for Q, one for K):                      */
/*      y_i = x_i * w_i / sqrt(mean_j x_j^2 + eps);                      */
/*  - RoPE rotates the pairs (i, i + D/2), i < D/2, by pos * theta_i,   */
/*    theta_i = base^(-2i/D): y_i = x_i c - x_{i+D/2} s,                */
/*    y_{i+D/2} = x_{i+D/2} c + x_i s;                                   */
/*  - the Hadamard rotation is y = H_D x / sqrt(D) with the Sylvester   */
/*    matrix H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]];               */
/*  - V is only quantised and stored;                                    */
/*  - a row's scale is amax / 448 (1 for an all-zero row) and its codes */
/*    are x / scale rounded to the nearest E4M3FN value, ties to the    */
/*    even code, saturating at +-448.                                    */
/* ------------------------------------------------------------------ */

/* Nearest E4M3FN code to v (ties to the code with an even mantissa,   */
/* |v| > 448 saturates), by comparing against every finite code.       */
int32_t orc_e4m3_encode(double v)
{
    int neg = v < 0 || (v == 0 && signbit(v));
    double a = fabs(v);
    if (a > 448.0)
        a = 448.0;
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c < 0x7F; ++c) { /* 0x00 .. 0x7E: the finite non-negative codes */
        double err = fabs(orc_e4m3_value(c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best_err = err;
            best = c;
        }
    }
    return neg ? (best | 0x80) : best;
}

/* Entry (i, j) of the Sylvester Hadamard matrix: (-1)^popcount(i & j). */
static int sylvester(int i, int j)
{
    return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1;
}

/* One head vector of D values: RMSNorm (if w), RoPE (if rope), Hadamard
 * (if hadamard), in that order.  In place. */
static void prologue_vector(double *x, int D, const float *w, double eps, int rope, double pos,
                            double base, int hadamard, double *tmp)
{
    if (w) {
        double ss = 0.0;
        for (int i = 0; i < D; ++i)
            ss += x[i] * x[i];
        double inv = 1.0 / sqrt(ss / D + eps);
        for (int i = 0; i < D; ++i)
            x[i] = x[i] * inv * (double)w[i];
    }
    if (rope) {
        int half = D / 2;
        for (int i = 0; i < half; ++i) {
            double theta = pos * pow(base, -2.0 * i / D);
            double c = cos(theta), s = sin(theta);
            double a = x[i], b = x[i + half];
            x[i] = a * c - b * s;
            x[i + half] = b * c + a * s;
        }
    }
    if (hadamard) {
        for (int i = 0; i < D; ++i) {
            double acc = 0.0;
            for (int j = 0; j < D; ++j)
                acc += sylvester(i, j) * x[j];
            tmp[i] = acc / sqrt((double)D);
        }
        memcpy(x, tmp, sizeof(double) * D);
    }
}

/* The prologue for T tokens.
 *   qkv       [T, (H_q + 2 H_kv) * D] bf16 bits: Q heads, then K, then V
 *   positions [T] int32, cache_slots [T] int32 (page * 64 + slot, or < 0:
 *             not stored)
 *   q_norm_w, k_norm_w [D] fp32 (NULL: no QK-Norm)
 * Outputs (fp64, before any rounding to the cache format):
 *   q_val [T, H_q, D], k_val [T, H_kv, D], v_val [T, H_kv, D]
 * and, for the fp8 format, per-row scales and codes:
 *   q_scale [T, H_q], k_scale / v_scale [T, H_kv], q_code [T, H_q, D],
 *   k_code / v_code [T, H_kv, D]  (any of these may be NULL). */
int orc_prologue(int32_t T, int32_t H_q, int32_t H_kv, int32_t D, const uint16_t *qkv,
                 const int32_t *positions, const float *q_norm_w, const float *k_norm_w,
                 double eps, int32_t rope, double rope_base, int32_t hadamard,
                 double *q_val, double *k_val, double *v_val,
                 double *q_scale, double *k_scale, double *v_scale,
                 uint8_t *q_code, uint8_t *k_code, uint8_t *v_code)
{
    const int heads = H_q + 2 * H_kv;
    int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
    for (int64_t th = 0; th < (int64_t)T * heads; ++th) {
        int t = (int)(th / heads), j = (int)(th % heads);
        double *x = (double *)malloc(sizeof(double) * D * 2);
        if (!x) {
            err |= 1;
            continue;
        }
        double *tmp = x + D;
        const uint16_t *src = qkv + ((int64_t)t * heads + j) * D;
        for (int i = 0; i < D; ++i)
            x[i] = orc_bf16_value(src[i]);
        int kind = j < H_q ? 0 : (j < H_q + H_kv ? 1 : 2);
        int hh = kind == 0 ? j : (kind == 1 ? j - H_q : j - H_q - H_kv);
        if (kind < 2)
            prologue_vector(x, D, kind == 0 ? q_norm_w : k_norm_w, eps, rope, positions[t],
                            rope_base, hadamard, tmp);
        double *val = kind == 0 ? q_val : (kind == 1 ? k_val : v_val);
        double *scl = kind == 0 ? q_scale : (kind == 1 ? k_scale : v_scale);
        uint8_t *code = kind == 0 ? q_code : (kind == 1 ? k_code : v_code);
        int64_t row = (int64_t)t * (kind == 0 ? H_q : H_kv) + hh;
        if (val)
            memcpy(val + row * D, x, sizeof(double) * D);
        double amax = 0.0;
        for (int i = 0; i < D; ++i)
            if (fabs(x[i]) > amax)
                amax = fabs(x[i]);
        double scale = amax > 0 ? amax / 448.0 : 1.0;
        if (scl)
            scl[row] = scale;
        if (code)
            for (int i = 0; i < D; ++i)
                code[row * D + i] = (uint8_t)orc_e4m3_encode(x[i] / scale);
        free(x);
    }
    return err ? -1 : 0;
}
