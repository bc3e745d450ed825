// Host-side argument validation of the C ABI, and the pure host queries
// (sizes, status strings, version).  No HIP here: see validate.h.
#include "validate.h"

#include <algorithm>

#include <math.h>

#include "layout.h"

namespace hpcattn {

bool sizes_ok(int32_t batch, int32_t num_kv_heads, int32_t num_bins) {
    return batch >= 1 && batch <= HPCATTN_MAX_BATCH && num_kv_heads >= 1 && num_bins >= 1 &&
           (int64_t)batch * num_kv_heads + num_bins - 1 <= INT32_MAX;
}

int64_t static_splits(int32_t policy, int32_t param, int32_t max_seq_len) {
    if (max_seq_len < 0 || param < 1) return -1;
    if (policy == 0) return param;
    if (policy == 1) {
        if (param % HPCATTN_PAGE_SIZE) return -1;
        const int64_t n = ((int64_t)max_seq_len + param - 1) / param;
        return n > 1 ? n : 1;
    }
    return -1;
}

int check_dims(const hpcattn_dims *d) {
    if (!d) return HPCATTN_ERR_NULL;
    // Every product below is taken in int64: a row count near 2^31 must not
    // wrap past the bound it is checked against.
    if (d->batch < 1 || d->batch > HPCATTN_MAX_BATCH || d->num_kv_heads < 1 ||
        d->num_q_heads < d->num_kv_heads || d->num_q_heads % d->num_kv_heads != 0 ||
        d->num_q_heads / d->num_kv_heads > HPCATTN_MAX_GROUP ||
        (d->head_dim != 64 && d->head_dim != 128) || d->max_pages_per_req < 1 ||
        d->num_pages < 1 || d->q_rows < 1 ||
        (int64_t)d->q_rows * (d->num_q_heads / d->num_kv_heads) > HPCATTN_MAX_ROWS)
        return HPCATTN_ERR_SHAPE;
    if (d->kv_dtype != HPCATTN_KV_BF16 && d->kv_dtype != HPCATTN_KV_FP8_E4M3)
        return HPCATTN_ERR_DTYPE;
    if (!isfinite(d->sm_scale)) return HPCATTN_ERR_ARG;
    return HPCATTN_OK;
}

int check_operands(const hpcattn_dims *d, const void *q, const float *q_scale,
                   const void *k_pages, const void *v_pages, const float *k_scale,
                   const float *v_scale, const int32_t *page_table) {
    if (!q || !k_pages || !v_pages || !page_table) return HPCATTN_ERR_NULL;
    const bool fp8 = d->kv_dtype == HPCATTN_KV_FP8_E4M3;
    const bool any_scale = q_scale || k_scale || v_scale;
    const bool all_scales = q_scale && k_scale && v_scale;
    if (fp8 ? !all_scales : any_scale) return HPCATTN_ERR_DTYPE;
    return HPCATTN_OK;
}

int check_map(const hpcattn_dims *d, const hpcattn_task_map *map) {
    if (!map || !map->words) return HPCATTN_ERR_NULL;
    if (!sizes_ok(map->batch, map->num_kv_heads, map->num_bins)) return HPCATTN_ERR_SHAPE;
    if (map->batch != d->batch || map->num_kv_heads != d->num_kv_heads) return HPCATTN_ERR_SHAPE;
    if (map->bytes < hpcattn_task_map_bytes(map->batch, map->num_kv_heads, map->num_bins))
        return HPCATTN_ERR_WORKSPACE;
    return HPCATTN_OK;
}

int check_plan(const int32_t *seq_lens, int32_t batch, int32_t num_kv_heads, int32_t num_bins,
               int32_t min_tiles, const hpcattn_task_map *map) {
    if (!seq_lens || !map || !map->words) return HPCATTN_ERR_NULL;
    if (!sizes_ok(batch, num_kv_heads, num_bins)) return HPCATTN_ERR_SHAPE;
    if (min_tiles < 1) return HPCATTN_ERR_ARG;
    if (map->bytes < hpcattn_task_map_bytes(batch, num_kv_heads, num_bins))
        return HPCATTN_ERR_WORKSPACE;
    return HPCATTN_OK;
}

// The checks decode and decode_combine share before their own buffers.
static int check_decode_inputs(const hpcattn_dims *d, const void *q, const float *q_scale,
                               const void *k_pages, const void *v_pages, const float *k_scale,
                               const float *v_scale, const int32_t *page_table,
                               const hpcattn_task_map *map) {
    int rc = check_dims(d);
    if (rc) return rc;
    rc = check_operands(d, q, q_scale, k_pages, v_pages, k_scale, v_scale, page_table);
    if (rc) return rc;
    return check_map(d, map);
}

int check_decode(const hpcattn_dims *d, const void *q, const float *q_scale,
                 const void *k_pages, const void *v_pages, const float *k_scale,
                 const float *v_scale, const int32_t *page_table, const hpcattn_task_map *map,
                 const float *part_o, const float *part_lse, int64_t part_o_rows) {
    const int rc = check_decode_inputs(d, q, q_scale, k_pages, v_pages, k_scale, v_scale,
                                       page_table, map);
    if (rc) return rc;
    if (!part_o || !part_lse) return HPCATTN_ERR_NULL;
    if (part_o_rows < hpcattn_max_partials(map->batch, map->num_kv_heads, map->num_bins))
        return HPCATTN_ERR_WORKSPACE;
    return HPCATTN_OK;
}

int check_decode_combine(const hpcattn_dims *d, const void *q, const float *q_scale,
                         const void *k_pages, const void *v_pages, const float *k_scale,
                         const float *v_scale, const int32_t *page_table,
                         const hpcattn_task_map *map, const float *part_o, const float *part_lse,
                         int64_t part_o_rows, const int32_t *tickets, int64_t num_tickets,
                         const void *out) {
    const int rc = check_decode_inputs(d, q, q_scale, k_pages, v_pages, k_scale, v_scale,
                                       page_table, map);
    if (rc) return rc;
    if (!part_o || !part_lse || !tickets || !out) return HPCATTN_ERR_NULL;
    if (part_o_rows < hpcattn_max_partials(map->batch, map->num_kv_heads, map->num_bins) ||
        num_tickets < (int64_t)map->batch * map->num_kv_heads)
        return HPCATTN_ERR_WORKSPACE;
    return HPCATTN_OK;
}

int check_combine(const hpcattn_dims *d, const hpcattn_task_map *map, const float *part_o,
                  const float *part_lse, const void *out) {
    int rc = check_dims(d);
    if (rc) return rc;
    rc = check_map(d, map);
    if (rc) return rc;
    if (!part_o || !part_lse || !out) return HPCATTN_ERR_NULL;
    return HPCATTN_OK;
}

int check_static(const hpcattn_dims *d, int32_t policy, int32_t param, int32_t max_seq_len,
                 const int32_t *seq_lens, const void *q, const float *q_scale,
                 const void *k_pages, const void *v_pages, const float *k_scale,
                 const float *v_scale, const int32_t *page_table, const float *part_o,
                 const float *part_lse, int64_t part_o_rows, const void *out) {
    int rc = check_dims(d);
    if (rc) return rc;
    rc = check_operands(d, q, q_scale, k_pages, v_pages, k_scale, v_scale, page_table);
    if (rc) return rc;
    if (!seq_lens || !part_o || !part_lse || !out) return HPCATTN_ERR_NULL;
    const int64_t splits = static_splits(policy, param, max_seq_len);
    if (splits < 1) return HPCATTN_ERR_ARG;
    // B H_kv splits workgroups, one partial slot each, addressed with int32
    // (divided, not multiplied: B H_kv splits can pass 2^63)
    const int64_t segs = (int64_t)d->batch * d->num_kv_heads;
    if (splits > INT32_MAX || segs > INT32_MAX / splits) return HPCATTN_ERR_SHAPE;
    if (part_o_rows < segs * splits) return HPCATTN_ERR_WORKSPACE;
    return HPCATTN_OK;
}

int check_probe(const void *buf, size_t bytes, int32_t workgroups, int32_t flags,
                const uint32_t *sink) {
    if (!buf || !sink) return HPCATTN_ERR_NULL;
    if (bytes < 16 || bytes % 16 || workgroups < 1 || (flags & ~3)) return HPCATTN_ERR_ARG;
    if (flags & 2) {   // a power-of-two number of 16 KB chunks
        const size_t n = bytes / 16384;
        if (bytes % 16384 || n == 0 || (n & (n - 1))) return HPCATTN_ERR_ARG;
    }
    return HPCATTN_OK;
}

int check_prologue(const hpcattn_prologue_dims *d, const void *qkv, const int32_t *positions,
                   const int32_t *cache_slots, const void *q_out, const float *q_scale,
                   const void *k_pages, const void *v_pages, const float *k_scale,
                   const float *v_scale) {
    if (!d) return HPCATTN_ERR_NULL;
    if (d->num_tokens < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
        (d->head_dim != 64 && d->head_dim != 128) || d->num_pages < 1)
        return HPCATTN_ERR_SHAPE;
    // The launch: one workgroup per token with one wave per 16 heads (at most
    // 16 waves); a grid's extent in work-items is 32-bit.
    const int64_t heads = (int64_t)d->num_q_heads + 2 * (int64_t)d->num_kv_heads;
    const int64_t waves = std::min<int64_t>((heads + 15) / 16, 16);
    if (heads > HPCATTN_PROLOGUE_MAX_HEADS || (int64_t)d->num_tokens * 64 * waves > UINT32_MAX)
        return HPCATTN_ERR_SHAPE;
    if (d->kv_dtype != HPCATTN_KV_BF16 && d->kv_dtype != HPCATTN_KV_FP8_E4M3)
        return HPCATTN_ERR_DTYPE;
    if ((d->flags & ~(HPCATTN_PROLOGUE_ROPE | HPCATTN_PROLOGUE_HADAMARD)) ||
        !(d->eps >= 0.f) || !isfinite(d->eps) || !(d->rope_base > 0.f) ||
        !isfinite(d->rope_base))
        return HPCATTN_ERR_ARG;
    const bool fp8 = d->kv_dtype == HPCATTN_KV_FP8_E4M3;
    if (d->num_tokens == 0) return HPCATTN_OK;   // nothing is read or written
    if (!qkv || !cache_slots || !q_out || !k_pages || !v_pages) return HPCATTN_ERR_NULL;
    if ((d->flags & HPCATTN_PROLOGUE_ROPE) && !positions) return HPCATTN_ERR_NULL;
    if (fp8 ? !(q_scale && k_scale && v_scale) : (q_scale || k_scale || v_scale))
        return HPCATTN_ERR_DTYPE;
    return HPCATTN_OK;
}

bool fuse_combine(const hpcattn_dims *d, const hpcattn_task_map *map) {
    // Fuse where it pays (measured): segments of a few chunks.  The last
    // workgroup of a segment merges its chunks alone, most often at the end
    // of the launch, so past a mean of 8 chunks (4 where a KV head serves
    // more than 16 query rows, whose partials are larger) decode and combine
    // run as two launches, with the same result.  Draft verification, 6 rows
    // of 8 heads: fused 300.5 vs 310.2 us at a mean of 2 chunks (bf16),
    // 388.1 vs 374.9 us at 5 (fp8).
    const int64_t S = (int64_t)map->batch * map->num_kv_heads;
    const int64_t mean_chunks = (S + map->num_bins - 1 + S - 1) / S;
    const int64_t rows = (int64_t)d->q_rows * (d->num_q_heads / d->num_kv_heads);
    return mean_chunks < (rows <= 16 ? 8 : 4);
}

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

ScratchPlan scratch_plan(const hpcattn_dims *d, const hpcattn_task_map *map) {
    ScratchPlan s{};
    const int64_t rg = (int64_t)d->q_rows * (d->num_q_heads / d->num_kv_heads);
    s.num_tickets = (int64_t)map->batch * map->num_kv_heads;
    s.rows = hpcattn_max_partials(map->batch, map->num_kv_heads, map->num_bins);
    s.lse = align256(4 * (int64_t)HPCATTN_NOALLOC_MAX_SEGMENTS);
    s.o = s.lse + align256(4 * s.rows * rg);
    s.end = s.o + 4 * s.rows * rg * d->head_dim;
    return s;
}

int check_decode_combine_noalloc(const hpcattn_dims *d, const void *q, const float *q_scale,
                                 const void *k_pages, const void *v_pages, const float *k_scale,
                                 const float *v_scale, const int32_t *page_table,
                                 const hpcattn_task_map *map, const void *out) {
    const int rc = check_decode_inputs(d, q, q_scale, k_pages, v_pages, k_scale, v_scale,
                                       page_table, map);
    if (rc) return rc;
    if (!out) return HPCATTN_ERR_NULL;
    const ScratchPlan s = scratch_plan(d, map);
    if (s.num_tickets > HPCATTN_NOALLOC_MAX_SEGMENTS ||
        s.end > (int64_t)HPCATTN_NOALLOC_SCRATCH_BYTES)
        return HPCATTN_ERR_WORKSPACE;
    return HPCATTN_OK;
}

}  // namespace hpcattn

extern "C" {

size_t hpcattn_task_map_bytes(int32_t batch, int32_t num_kv_heads, int32_t num_bins) {
    if (batch < 1 || num_kv_heads < 1 || num_bins < 1) return 0;
    return (size_t)hpcattn::MapLayout(batch, num_kv_heads, num_bins).words * sizeof(int32_t);
}

int64_t hpcattn_max_partials(int32_t batch, int32_t num_kv_heads, int32_t num_bins) {
    if (batch < 1 || num_kv_heads < 1 || num_bins < 1) return 0;
    return (int64_t)batch * num_kv_heads + num_bins - 1;
}

int64_t hpcattn_static_max_partials(int32_t batch, int32_t num_kv_heads, int32_t policy,
                                    int32_t param, int32_t max_seq_len) {
    if (batch < 1 || num_kv_heads < 1) return 0;
    const int64_t splits = hpcattn::static_splits(policy, param, max_seq_len);
    const int64_t segs = (int64_t)batch * num_kv_heads;
    if (splits < 1 || segs > INT32_MAX / splits) return 0;   // more rows than int32 slots
    return segs * splits;
}

const char *hpcattn_strerror(int status) {
    switch (status) {
    case HPCATTN_OK: return "ok";
    case HPCATTN_ERR_NULL: return "a required pointer is NULL";
    case HPCATTN_ERR_SHAPE: return "a size is out of range or inconsistent";
    case HPCATTN_ERR_DTYPE: return "unknown KV dtype, or scales given for bf16 / missing for fp8";
    case HPCATTN_ERR_WORKSPACE:
        return "a caller buffer (or the fixed scratch of the allocation-free call) is too small";
    case HPCATTN_ERR_LAUNCH: return "the HIP runtime reported a launch error";
    case HPCATTN_ERR_ARG: return "an argument is out of range";
    default: return "unknown status";
    }
}

int hpcattn_version(void) { return 200; }

}  // extern "C"
