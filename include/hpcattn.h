/*
 * hpcattn.h -- C ABI of load-balanced split-KV decode attention over a paged
 * GQA KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The method ("HPC-Ops x SGLang: Tencent Hunyuan open-sources high-performance
 * Attention, Router GEMM and MoE operators", sections "Attention: load
 * balancing for variable-length decode" and "Scheduling around live KV work";
 * "Hy3 preview full-stack inference optimization", section 2.1.1 "Attention
 * dynamic scheduling"):
 *
 *   1. hpcattn_plan     once per decode step: cut each request's live KV into
 *                       64-token tiles, count them over all requests and KV
 *                       heads, split the total into near-equal bins, one per
 *                       persistent workgroup, and write the task map.
 *   2. hpcattn_decode   per layer: each persistent workgroup drains its bin
 *                       and writes one partial output with its log-sum-exp
 *                       per descriptor.
 *   3. hpcattn_combine  per layer: merge each (request, KV head)'s partials
 *                       under the global softmax.
 *   hpcattn_decode_combine does 2 and 3 in one launch.
 *   hpcattn_static_decode is the static split-KV scheme the pages compare
 *   against (fixed split count, or fixed chunk size), for ablation.
 *
 * Multi-row decode ("Hy3 preview full-stack inference optimization", section
 * 2.5, MTP; "SGLang Low-Latency Mode: Kernels and Runtime", section 1: a
 * verify step checks the confirmed token and the draft tokens of a request
 * in one forward): with q_rows = R > 1 each request brings R query rows, the
 * last R tokens of the request, which the cache already holds.  Row r sits
 * at position L_b - R + r and attends to tokens [0, L_b - R + r] (a causal
 * mask among the rows; the pages give none, this is the plain reading of
 * verifying a token sequence).  The plan and its task map do not change:
 * one K/V tile serves all R G rows of its KV head.  R = 1 is plain decode.
 *
 * Conventions (all entry points):
 *   - Every pointer argument is a DEVICE pointer unless marked "host".
 *   - The caller owns every buffer.  The library allocates and frees
 *     nothing, keeps no state between calls (beyond kernel attributes it
 *     reads once from the runtime), never synchronises and never copies
 *     between host and device.  Work is enqueued on `stream` (a hipStream_t;
 *     NULL is the default stream) and is safe to capture in a HIP graph.
 *   - Return 0 (HPCATTN_OK) or a negative hpcattn_status.  Argument errors
 *     are detected on the host before anything is enqueued; a launch error
 *     reported by the runtime returns HPCATTN_ERR_LAUNCH.
 *   - Layouts are row-major and contiguous:
 *       q           [B, R, H_q, D]           bf16, or e4m3 bytes
 *       q_scale     [B, R, H_q]              fp32 (fp8 only)
 *       k_pages     [num_pages, H_kv, 64, D] bf16, or e4m3 bytes
 *       v_pages     [num_pages, H_kv, 64, D] same type as k_pages
 *       k_scale     [num_pages, H_kv, 64]    fp32 (fp8 only); v_scale likewise
 *       page_table  [B, max_pages_per_req]   int32; token t of request b sits
 *                   in slot t % 64 of page page_table[b][t / 64]
 *       part_o      [max_partials, R G, D]   fp32, normalised partial output;
 *                   row r G + g is query row r, head h G + g
 *       part_lse    [max_partials, R G]      fp32, natural-log LSE of the
 *                   scaled logits of the partial's tokens
 *       out         [B, R, H_q, D]           bf16 (round to nearest even)
 *       out_lse     [B, R, H_q]              fp32, natural log
 *     R = q_rows (the R axis is absent in effect when R = 1);
 *     G = H_q / H_kv; query head j reads KV head j / G.  fp8 is OCP E4M3FN
 *     and a value is code * scale.
 *   - Data errors (a length beyond 64 * max_pages_per_req, a page id outside
 *     [0, num_pages)) never fault: out-of-range tiles are skipped and their
 *     tokens contribute nothing; plan sets the map's error word.
 */
#ifndef HPCATTN_H
#define HPCATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HPCATTN_PAGE_SIZE 64   /* tokens per KV page and per tile            */
#define HPCATTN_MAX_BATCH 8192 /* requests per plan                          */
#define HPCATTN_MAX_GROUP 16   /* query heads per KV head                     */
#define HPCATTN_MAX_ROWS 64    /* query rows per KV head, q_rows * G          */

typedef enum {
    HPCATTN_OK = 0,
    HPCATTN_ERR_NULL = -1,      /* a required pointer is NULL                  */
    HPCATTN_ERR_SHAPE = -2,     /* a size is out of range or inconsistent      */
    HPCATTN_ERR_DTYPE = -3,     /* unknown dtype, or scales given/missing      */
    HPCATTN_ERR_WORKSPACE = -4, /* a buffer (caller's or fixed scratch) too small */
    HPCATTN_ERR_LAUNCH = -5,    /* the HIP runtime reported a launch error     */
    HPCATTN_ERR_ARG = -6        /* another argument is out of range            */
} hpcattn_status;

typedef enum {
    HPCATTN_KV_BF16 = 0,        /* q, k_pages, v_pages in bf16                 */
    HPCATTN_KV_FP8_E4M3 = 1     /* OCP E4M3FN bytes with fp32 scales           */
} hpcattn_kv_dtype;

/* Error word (map header word 7) values written by hpcattn_plan. */
#define HPCATTN_MAPERR_NEG_LEN 1   /* a sequence length < 0 (taken as 0)      */
#define HPCATTN_MAPERR_OVERFLOW 2  /* more than 2^31 - 1 tiles in the batch   */

/* Problem shape of one attention layer (host struct). */
typedef struct {
    int32_t batch;              /* B >= 1                                      */
    int32_t num_q_heads;        /* H_q, a multiple of H_kv                     */
    int32_t num_kv_heads;       /* H_kv >= 1; G = H_q / H_kv <= 16             */
    int32_t head_dim;           /* D, 64 or 128                                */
    int32_t max_pages_per_req;  /* columns of page_table                       */
    int32_t num_pages;          /* pages in k_pages / v_pages                  */
    int32_t kv_dtype;           /* hpcattn_kv_dtype                            */
    float sm_scale;             /* softmax scale on q . k, e.g. 1/sqrt(D)      */
    int32_t q_rows;             /* R >= 1 query rows per request (1 + drafts); */
                                /* q_rows * G <= HPCATTN_MAX_ROWS              */
} hpcattn_dims;

/*
 * Task map handle (host struct describing a device buffer).
 *
 * The device buffer holds int32 words:
 *   [0..7]  header {T, P_eff, q, r, num_desc, B, H_kv, err}
 *   then    seq_lens[B]                      copy of the planned lengths
 *           bin_desc_off[P + 1]              descriptors of bin i are
 *                                            bin_desc_off[i] .. [i + 1] - 1
 *           seg_desc_off[B * H_kv + 1]       descriptors of segment
 *                                            s = b * H_kv + h, contiguous
 *           desc[B * H_kv + P - 1][4]        {b, h, t0, t1}: tiles [t0, t1)
 *                                            of segment (b, h); unused
 *                                            entries are zero
 * T is the total tile count, P_eff the bins in use, and bins 0 .. r - 1 own
 * q + 1 tiles, bins r .. P_eff - 1 own q, the rest none.  A descriptor's
 * index is its partial slot in part_o / part_lse.
 */
typedef struct {
    int32_t *words;             /* device, hpcattn_task_map_bytes() bytes      */
    size_t bytes;               /* size of `words` in bytes                    */
    int32_t batch;              /* B the map was planned for                   */
    int32_t num_kv_heads;       /* H_kv                                        */
    int32_t num_bins;           /* P = num_persistent_wg                       */
    int32_t min_tiles;          /* minimum-work floor m                        */
} hpcattn_task_map;

/* Bytes of the task map buffer for (B, H_kv, P); 0 if a size is < 1. */
size_t hpcattn_task_map_bytes(int32_t batch, int32_t num_kv_heads, int32_t num_bins);

/* Partial slots a plan can produce: B * H_kv + P - 1 (part_o / part_lse
 * leading dimension); 0 if a size is < 1. */
int64_t hpcattn_max_partials(int32_t batch, int32_t num_kv_heads, int32_t num_bins);

/*
 * The number of decode workgroups that are co-resident on the current device
 * (compute units x workgroups per CU at the kernel's register and LDS use)
 * for this head_dim, kv_dtype and rows = q_rows * G query rows per KV head
 * (G for plain decode): the natural num_bins, one
 * persistent workgroup per bin with no second round.  A host query (reads
 * device attributes, enqueues nothing).  Returns > 0, or HPCATTN_ERR_ARG for
 * an unsupported shape, HPCATTN_ERR_LAUNCH if the runtime cannot answer.
 */
int32_t hpcattn_suggest_num_bins(int32_t head_dim, int32_t kv_dtype, int32_t rows);

/*
 * The assign step ("Scheduling around live KV work"; "Attention dynamic
 * scheduling": the task map is built before each step from device-side
 * lengths and every layer's attention takes its tasks from it).
 *
 * seq_lens   device int32 [batch], live KV tokens per request.
 * num_bins   P >= 1, the number of persistent workgroups of hpcattn_decode.
 * min_tiles  m >= 1, minimum-work floor: at most max(1, T / m) bins are used,
 *            so each used bin owns >= m tiles when T >= m.
 * map        host struct: in `words`/`bytes` (device buffer, at least
 *            hpcattn_task_map_bytes(batch, num_kv_heads, num_bins) bytes);
 *            out: the other fields.  One workgroup of 1024 threads writes the
 *            whole buffer.  Deterministic: the words are a pure function of
 *            (seq_lens, num_kv_heads, num_bins, min_tiles).
 * Errors: NULL pointers, batch outside [1, HPCATTN_MAX_BATCH], H_kv < 1,
 * P < 1, m < 1, a buffer smaller than required.
 */
int hpcattn_plan(const int32_t *seq_lens, int32_t batch, int32_t num_kv_heads,
                 int32_t num_bins, int32_t min_tiles, hpcattn_task_map *map,
                 void *stream);

/*
 * The persistent decode step ("Scheduling around live KV work": each
 * workgroup drains its bin, computing attention over one or more contiguous
 * KV tiles per descriptor and writing a partial output with its log-sum-exp).
 *
 * Launches map->num_bins workgroups, bin i drained by workgroup i: 256
 * threads, or when q_rows * G > 16 64 per 16 query rows of a KV head (plus
 * a 64-thread staging wave for 33 .. 48 rows at head_dim 128).  Writes
 * part_o / part_lse rows 0 .. num_desc - 1 and nothing else.  dims->batch
 * and dims->num_kv_heads must equal the map's.
 * q_scale, k_scale, v_scale: NULL for bf16, required for fp8.
 * part_o / part_lse: at least hpcattn_max_partials(B, H_kv, P) rows;
 * part_o_rows gives the caller's row capacity.
 */
int hpcattn_decode(const hpcattn_dims *dims, const void *q, const float *q_scale,
                   const void *k_pages, const void *v_pages,
                   const float *k_scale, const float *v_scale,
                   const int32_t *page_table, const hpcattn_task_map *map,
                   float *part_o, float *part_lse, int64_t part_o_rows,
                   void *stream);

/*
 * The combine step ("Scheduling around live KV work": a final kernel reads
 * each request's and head's actual chunk count and merges the partials under
 * the global softmax normalisation; "Attention dynamic scheduling": the
 * Combine kernel merges the split-KV results).
 *
 * For segment s = (b, h) with partials k in seg_desc_off[s] .. [s + 1] - 1:
 *   M = max_k lse_k,  w_k = exp(lse_k - M),
 *   out = sum_k w_k o_k / sum_k w_k,  out_lse = M + ln sum_k w_k.
 * A request with no live KV gets out = 0 and out_lse = -inf.
 * out_lse may be NULL.
 */
int hpcattn_combine(const hpcattn_dims *dims, const hpcattn_task_map *map,
                    const float *part_o, const float *part_lse, void *out,
                    float *out_lse, void *stream);

/*
 * Decode and combine in one launch: the same result as hpcattn_decode
 * followed by hpcattn_combine, with one kernel per layer instead of two
 * ("SGLang Low-Latency Mode: Kernels and Runtime", section 3: each small
 * kernel costs its launch and its tail even under HIP graphs).
 *
 * A segment cut into one chunk writes its out rows directly.  Otherwise
 * each workgroup that finishes a chunk writes its partial with the
 * device-coherent cache policy and increments tickets[b * H_kv + h]; the
 * workgroup that takes the last ticket merges the segment's partials as
 * hpcattn_combine does (up to summation order) and resets the ticket to 0.
 * No workgroup ever waits for another.  Where fusing does not pay -- a mean
 * of 8 or more chunks per segment (S + P - 1 descriptors over S = B H_kv
 * segments; 4 or more when q_rows * G > 16), or a shape whose fused kernel
 * holds fewer workgroups per CU than hpcattn_decode's -- the call runs
 * hpcattn_decode and hpcattn_combine instead, with the same result.
 *
 * tickets: device int32 [num_tickets >= B * H_kv], all zero on entry; the
 *   call leaves them zero.  Zero them once after allocating; reuse freely
 *   across layers and steps.  Calls that share a tickets buffer must not
 *   overlap.
 * part_o / part_lse: scratch for the multi-chunk segments, sized as for
 *   hpcattn_decode.  out / out_lse: as for hpcattn_combine (out_lse may be
 *   NULL).  Errors as for hpcattn_decode, plus NULL tickets / out and
 *   num_tickets < B * H_kv (HPCATTN_ERR_WORKSPACE).
 */
int hpcattn_decode_combine(const hpcattn_dims *dims, const void *q, const float *q_scale,
                           const void *k_pages, const void *v_pages,
                           const float *k_scale, const float *v_scale,
                           const int32_t *page_table, const hpcattn_task_map *map,
                           float *part_o, float *part_lse, int64_t part_o_rows,
                           int32_t *tickets, int64_t num_tickets, void *out,
                           float *out_lse, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): the same call
 * as hpcattn_decode_combine, with the same result, whose partials and
 * tickets live in a fixed scratch array that the library holds on each
 * device it runs on, from the first call until the process ends.  The
 * caller passes inputs, the task map and out / out_lse only.
 *
 * Limits: B * H_kv <= HPCATTN_NOALLOC_MAX_SEGMENTS, and the partials,
 * hpcattn_max_partials(B, H_kv, P) rows of R G (D + 1) fp32 values (each
 * block 256-byte aligned), fit in HPCATTN_NOALLOC_SCRATCH_BYTES after the
 * ticket block; otherwise HPCATTN_ERR_WORKSPACE and nothing is enqueued.
 * The call allocates and frees nothing.  Its first call on a device looks
 * up that device's array and enqueues one small kernel that zeroes the
 * tickets (static storage starts at zero too); every call leaves them zero.
 * Every call on one device shares that device's array: calls that may
 * overlap on one device (other streams, concurrent graphs) race and must be
 * ordered by the caller.  Errors as for hpcattn_decode_combine, plus
 * HPCATTN_ERR_LAUNCH when the runtime cannot name the array's address.
 */
#define HPCATTN_NOALLOC_SCRATCH_BYTES (32u << 20)   /* per device               */
#define HPCATTN_NOALLOC_MAX_SEGMENTS 65536          /* B * H_kv                 */

int hpcattn_decode_combine_noalloc(const hpcattn_dims *dims, const void *q, const float *q_scale,
                                   const void *k_pages, const void *v_pages,
                                   const float *k_scale, const float *v_scale,
                                   const int32_t *page_table, const hpcattn_task_map *map,
                                   void *out, float *out_lse, void *stream);

/*
 * Static split-KV decode, the scheme the dynamic one replaces ("Attention:
 * load balancing for variable-length decode": a fixed launch grid over KV
 * heads, requests and KV chunks with one partition policy for the batch).
 *
 * policy 0, fixed split count: param = S >= 1 splits per (request, KV head);
 *   split k of a request with n tiles owns tiles [k n / S, (k + 1) n / S).
 * policy 1, fixed chunk size: param = C tokens, a positive multiple of 64;
 *   the grid reserves ceil(max_seq_len / C) chunks per (request, KV head)
 *   and chunk k owns tokens [k C, (k + 1) C) clipped to the length.
 * max_seq_len (host) bounds every seq_lens[b] and sizes the policy-1 grid.
 * One workgroup per (request, KV head, split), of the same size as the
 * dynamic decode's; empty splits write lse = -inf.  Then the combine runs over the fixed splits and writes
 * out / out_lse like hpcattn_combine.  part_o / part_lse need
 * hpcattn_static_max_partials() rows (given in part_o_rows).
 */
int hpcattn_static_decode(const hpcattn_dims *dims, int32_t policy, int32_t param,
                          int32_t max_seq_len, const int32_t *seq_lens,
                          const void *q, const float *q_scale,
                          const void *k_pages, const void *v_pages,
                          const float *k_scale, const float *v_scale,
                          const int32_t *page_table, float *part_o, float *part_lse,
                          int64_t part_o_rows, void *out, float *out_lse,
                          void *stream);

/* Partial rows hpcattn_static_decode needs: B * H_kv * splits, where splits
 * is S (policy 0) or ceil(max_seq_len / C) (policy 1); 0 on bad input or
 * when that exceeds INT32_MAX rows (hpcattn_static_decode rejects it). */
int64_t hpcattn_static_max_partials(int32_t batch, int32_t num_kv_heads, int32_t policy,
                                    int32_t param, int32_t max_seq_len);

/*
 * Measurement reference, not part of the method: a plain streaming read of
 * `bytes` (a positive multiple of 16) from device buffer `buf`, 16-byte loads
 * in a grid-stride loop over `workgroups` workgroups of 256 threads; flags
 * bit 0 selects nontemporal loads (the form the decode kernel uses for KV);
 * bit 1 reads the buffer as 16 KB chunks in a scattered order (the shape of
 * the decode kernel's shuffled tiles; `bytes` must then be a power-of-two
 * number of 16 KB chunks); other bits must be 0.  It writes nothing but (practically never) one word
 * of `sink` (device, 4 bytes).
 * Timing it gives the achievable HBM read bandwidth that the decode kernel's
 * bandwidth is compared with.
 */
int hpcattn_probe_stream_read(const void *buf, size_t bytes, int32_t workgroups, int32_t flags,
                              uint32_t *sink, void *stream);

/* Prologue limits: H_q + 2 H_kv heads at most, and T * 64 * min(ceil((H_q +
 * 2 H_kv) / 16), 16) below 2^32 (one workgroup per token with one wave per
 * 16 heads; at 256 heads or more, T below 4194304). */
#define HPCATTN_PROLOGUE_MAX_HEADS 65536

/* Prologue flags. */
#define HPCATTN_PROLOGUE_ROPE 1      /* rotate Q and K by their positions      */
#define HPCATTN_PROLOGUE_HADAMARD 2  /* rotate Q and K by H_D / sqrt(D)         */

/* Shape and options of one prologue call (host struct). */
typedef struct {
    int32_t num_tokens;         /* T >= 0 tokens (one per request in decode)  */
    int32_t num_q_heads;        /* H_q >= 1                                   */
    int32_t num_kv_heads;       /* H_kv >= 1                                  */
    int32_t head_dim;           /* D, 64 or 128                               */
    int32_t num_pages;          /* pages in k_pages / v_pages                 */
    int32_t kv_dtype;           /* HPCATTN_KV_BF16 or HPCATTN_KV_FP8_E4M3     */
    int32_t flags;              /* HPCATTN_PROLOGUE_* bits                    */
    float eps;                  /* RMSNorm epsilon, >= 0                      */
    float rope_base;            /* RoPE base (e.g. 10000), > 0                */
} hpcattn_prologue_dims;

/*
 * The attention prologue, fused ("Fused attention prologue": QK-Norm before
 * RoPE, Q in FP8 with per-token per-head scales passed to attention as is,
 * K and V written straight into the paged FP8 cache; "Hy3 preview full-stack
 * inference optimization" 2.2.1: RoPE + RMSNorm + optional Hadamard +
 * quantisation + KV store in one kernel).  For each token t and head:
 *   Q, K:  x <- x * w / sqrt(mean(x^2) + eps)        (if q_norm_w / k_norm_w)
 *          (x_i, x_{i+D/2}) rotated by positions[t] * base^(-2i/D)  (ROPE)
 *          x <- H_D x / sqrt(D), Sylvester H_D                       (HADAMARD)
 *   V:     unchanged.
 * Outputs, bf16 format: q_out [T, H_q, D] bf16; K, V rows into the bf16
 * cache.  fp8 format: each row (one token, one head) gets scale
 * amax / 448 (1 if all zero) and codes RNE(x / scale) in OCP E4M3FN:
 * q_out [T, H_q, D] bytes + q_scale [T, H_q]; K, V rows + k_scale, v_scale
 * entries in the paged cache and its scale pools.
 *
 * qkv          device bf16 [T, (H_q + 2 H_kv) * D]: Q heads, then K, then V
 * positions    device int32 [T] (needed with ROPE, else may be NULL)
 * cache_slots  device int32 [T]: page * 64 + slot of token t's K/V in the
 *              cache; a negative slot (or a page >= num_pages) stores nothing
 * q_norm_w, k_norm_w  device fp32 [D] or NULL (no QK-Norm)
 * q_scale, k_scale, v_scale: required for fp8, NULL for bf16.
 * Writes only q_out/q_scale rows of the T tokens and the cache rows named by
 * cache_slots.  With T = 0 nothing is read or written and the buffer
 * pointers may be NULL.  Errors: NULL pointers, sizes out of range (see the
 * prologue limits above), unknown flags or dtype, eps < 0, rope_base <= 0.
 */
int hpcattn_prologue(const hpcattn_prologue_dims *dims, const void *qkv,
                     const int32_t *positions, const int32_t *cache_slots,
                     const float *q_norm_w, const float *k_norm_w, void *q_out, float *q_scale,
                     void *k_pages, void *v_pages, float *k_scale, float *v_scale,
                     void *stream);

/* Static description of a status code (host string, never NULL). */
const char *hpcattn_strerror(int status);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int hpcattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HPCATTN_H */
