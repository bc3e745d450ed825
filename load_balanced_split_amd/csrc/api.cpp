// C ABI of libhpcattn: argument validation on the host, then the launches.
// Every check runs before anything is enqueued, so a rejected call has no
// side effect.  See hpcattn.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "common.h"
#include "hpcattn.h"

using namespace hpcattn;

namespace {

constexpr float kLog2e = 1.4426950408889634f;

int launch_status(hipError_t e) { return e == hipSuccess ? HPCATTN_OK : HPCATTN_ERR_LAUNCH; }

bool sizes_ok(int32_t batch, int32_t num_kv_heads, int32_t num_bins) {
    return batch >= 1 && batch <= HPCATTN_MAX_BATCH && num_kv_heads >= 1 && num_bins >= 1 &&
           (int64_t)batch * num_kv_heads + num_bins - 1 <= INT32_MAX;
}

int check_dims(const hpcattn_dims *d) {
    if (!d) return HPCATTN_ERR_NULL;
    if (d->batch < 1 || d->batch > HPCATTN_MAX_BATCH || d->num_kv_heads < 1 ||
        d->num_q_heads < d->num_kv_heads || d->num_q_heads % d->num_kv_heads != 0 ||
        d->num_q_heads / d->num_kv_heads > HPCATTN_MAX_GROUP ||
        (d->head_dim != 64 && d->head_dim != 128) || d->max_pages_per_req < 1 ||
        d->num_pages < 1 || d->q_rows < 1 ||
        d->q_rows * (d->num_q_heads / d->num_kv_heads) > HPCATTN_MAX_ROWS)
        return HPCATTN_ERR_SHAPE;
    if (d->kv_dtype != HPCATTN_KV_BF16 && d->kv_dtype != HPCATTN_KV_FP8_E4M3)
        return HPCATTN_ERR_DTYPE;
    if (!std::isfinite(d->sm_scale)) return HPCATTN_ERR_ARG;
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

DecodeParams make_params(const hpcattn_dims *d, const void *q, const float *q_scale,
                         const void *k_pages, const void *v_pages, const float *k_scale,
                         const float *v_scale, const int32_t *page_table, float *part_o,
                         float *part_lse) {
    DecodeParams p{};
    p.q = q;
    p.q_scale = q_scale;
    p.k = k_pages;
    p.v = v_pages;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.page_table = page_table;
    p.part_o = part_o;
    p.part_lse = part_lse;
    p.B = d->batch;
    p.Hq = d->num_q_heads;
    p.Hkv = d->num_kv_heads;
    p.G = d->num_q_heads / d->num_kv_heads;
    p.max_pages = d->max_pages_per_req;
    p.num_pages = d->num_pages;
    p.R = d->q_rows;
    p.scale_log2 = d->sm_scale * kLog2e;
    return p;
}

int64_t static_splits(int32_t policy, int32_t param, int32_t max_seq_len) {
    if (max_seq_len < 0 || param < 1) return -1;
    if (policy == 0) return param;
    if (policy == 1) {
        if (param % HPCATTN_PAGE_SIZE) return -1;
        return std::max<int64_t>(1, ((int64_t)max_seq_len + param - 1) / param);
    }
    return -1;
}

int check_map(const hpcattn_dims *d, const hpcattn_task_map *map) {
    if (!map || !map->words) return HPCATTN_ERR_NULL;
    if (!sizes_ok(map->batch, map->num_kv_heads, map->num_bins)) return HPCATTN_ERR_SHAPE;
    if (map->batch != d->batch || map->num_kv_heads != d->num_kv_heads) return HPCATTN_ERR_SHAPE;
    if (map->bytes < hpcattn_task_map_bytes(map->batch, map->num_kv_heads, map->num_bins))
        return HPCATTN_ERR_WORKSPACE;
    return HPCATTN_OK;
}

}  // namespace

extern "C" {

size_t hpcattn_task_map_bytes(int32_t batch, int32_t num_kv_heads, int32_t num_bins) {
    if (batch < 1 || num_kv_heads < 1 || num_bins < 1) return 0;
    return (size_t)MapLayout(batch, num_kv_heads, num_bins).words * sizeof(int32_t);
}

int64_t hpcattn_max_partials(int32_t batch, int32_t num_kv_heads, int32_t num_bins) {
    if (batch < 1 || num_kv_heads < 1 || num_bins < 1) return 0;
    return (int64_t)batch * num_kv_heads + num_bins - 1;
}

int hpcattn_plan(const int32_t *seq_lens, int32_t batch, int32_t num_kv_heads,
                 int32_t num_bins, int32_t min_tiles, hpcattn_task_map *map, void *stream) {
    if (!seq_lens || !map || !map->words) return HPCATTN_ERR_NULL;
    if (!sizes_ok(batch, num_kv_heads, num_bins)) return HPCATTN_ERR_SHAPE;
    if (min_tiles < 1) return HPCATTN_ERR_ARG;
    if (map->bytes < hpcattn_task_map_bytes(batch, num_kv_heads, num_bins))
        return HPCATTN_ERR_WORKSPACE;
    const hipError_t e = launch_plan(seq_lens, batch, num_kv_heads, num_bins, min_tiles,
                                     map->words, (hipStream_t)stream);
    if (e != hipSuccess) return HPCATTN_ERR_LAUNCH;
    map->batch = batch;
    map->num_kv_heads = num_kv_heads;
    map->num_bins = num_bins;
    map->min_tiles = min_tiles;
    return HPCATTN_OK;
}

int hpcattn_decode(const hpcattn_dims *dims, const void *q, const float *q_scale,
                   const void *k_pages, const void *v_pages, const float *k_scale,
                   const float *v_scale, const int32_t *page_table,
                   const hpcattn_task_map *map, float *part_o, float *part_lse,
                   int64_t part_o_rows, void *stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    rc = check_operands(dims, q, q_scale, k_pages, v_pages, k_scale, v_scale, page_table);
    if (rc) return rc;
    rc = check_map(dims, map);
    if (rc) return rc;
    if (!part_o || !part_lse) return HPCATTN_ERR_NULL;
    if (part_o_rows < hpcattn_max_partials(map->batch, map->num_kv_heads, map->num_bins))
        return HPCATTN_ERR_WORKSPACE;
    DecodeParams p = make_params(dims, q, q_scale, k_pages, v_pages, k_scale, v_scale,
                                 page_table, part_o, part_lse);
    p.map = map->words;
    p.P = map->num_bins;
    return launch_status(launch_decode(p, dims->head_dim, dims->kv_dtype, (hipStream_t)stream));
}

int hpcattn_decode_combine(const hpcattn_dims *dims, const void *q, const float *q_scale,
                           const void *k_pages, const void *v_pages, const float *k_scale,
                           const float *v_scale, const int32_t *page_table,
                           const hpcattn_task_map *map, float *part_o, float *part_lse,
                           int64_t part_o_rows, int32_t *tickets, int64_t num_tickets, void *out,
                           float *out_lse, void *stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    rc = check_operands(dims, q, q_scale, k_pages, v_pages, k_scale, v_scale, page_table);
    if (rc) return rc;
    rc = check_map(dims, map);
    if (rc) return rc;
    if (!part_o || !part_lse || !tickets || !out) return HPCATTN_ERR_NULL;
    if (part_o_rows < hpcattn_max_partials(map->batch, map->num_kv_heads, map->num_bins) ||
        num_tickets < (int64_t)map->batch * map->num_kv_heads)
        return HPCATTN_ERR_WORKSPACE;
    DecodeParams p = make_params(dims, q, q_scale, k_pages, v_pages, k_scale, v_scale,
                                 page_table, part_o, part_lse);
    p.map = map->words;
    p.P = map->num_bins;
    // Fuse where it pays (measured): segments of a few chunks on the per-wave
    // kernel.  Long segments (a mean of >= 8 chunks: the last workgroup would
    // merge many partials alone) and workgroups of more than 16 query rows run
    // decode and combine as two launches, with the same result.
    const int64_t S = (int64_t)map->batch * map->num_kv_heads;
    const int64_t mean_chunks = (S + map->num_bins - 1 + S - 1) / S;
    const int rows = dims->q_rows * (dims->num_q_heads / dims->num_kv_heads);
    if (mean_chunks >= 8 || rows > 16) {
        hipError_t e = launch_decode(p, dims->head_dim, dims->kv_dtype, (hipStream_t)stream);
        if (e != hipSuccess) return HPCATTN_ERR_LAUNCH;
        return hpcattn_combine(dims, map, part_o, part_lse, out, out_lse, stream);
    }
    p.out = out;
    p.out_lse = out_lse;
    p.tickets = tickets;
    return launch_status(launch_decode(p, dims->head_dim, dims->kv_dtype, (hipStream_t)stream));
}

int hpcattn_combine(const hpcattn_dims *dims, const hpcattn_task_map *map,
                    const float *part_o, const float *part_lse, void *out, float *out_lse,
                    void *stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    rc = check_map(dims, map);
    if (rc) return rc;
    if (!part_o || !part_lse || !out) return HPCATTN_ERR_NULL;
    CombineParams c{};
    c.part_o = part_o;
    c.part_lse = part_lse;
    c.seg_off = map->words + MapLayout(map->batch, map->num_kv_heads, map->num_bins).seg_off;
    c.stride = 0;
    c.out = out;
    c.out_lse = out_lse;
    c.S = dims->batch * dims->num_kv_heads;
    c.G = dims->num_q_heads / dims->num_kv_heads;
    c.D = dims->head_dim;
    c.R = dims->q_rows;
    c.Hkv = dims->num_kv_heads;
    c.max_chunks = hpcattn_max_partials(map->batch, map->num_kv_heads, map->num_bins);
    return launch_status(launch_combine(c, (hipStream_t)stream));
}

int32_t hpcattn_suggest_num_bins(int32_t head_dim, int32_t kv_dtype, int32_t rows) {
    if ((head_dim != 64 && head_dim != 128) || rows < 1 || rows > HPCATTN_MAX_ROWS ||
        (kv_dtype != HPCATTN_KV_BF16 && kv_dtype != HPCATTN_KV_FP8_E4M3))
        return HPCATTN_ERR_ARG;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return HPCATTN_ERR_LAUNCH;
    const int32_t per_cu = decode_resident_per_cu(head_dim, kv_dtype, rows);
    if (per_cu < 1 || cus < 1) return HPCATTN_ERR_LAUNCH;
    return per_cu * cus;
}

int64_t hpcattn_static_max_partials(int32_t batch, int32_t num_kv_heads, int32_t policy,
                                    int32_t param, int32_t max_seq_len) {
    if (batch < 1 || num_kv_heads < 1) return 0;
    const int64_t splits = static_splits(policy, param, max_seq_len);
    if (splits < 1) return 0;
    return (int64_t)batch * num_kv_heads * splits;
}

int hpcattn_static_decode(const hpcattn_dims *dims, int32_t policy, int32_t param,
                          int32_t max_seq_len, const int32_t *seq_lens, const void *q,
                          const float *q_scale, const void *k_pages, const void *v_pages,
                          const float *k_scale, const float *v_scale,
                          const int32_t *page_table, float *part_o, float *part_lse,
                          int64_t part_o_rows, void *out, float *out_lse, void *stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    rc = check_operands(dims, q, q_scale, k_pages, v_pages, k_scale, v_scale, page_table);
    if (rc) return rc;
    if (!seq_lens || !part_o || !part_lse || !out) return HPCATTN_ERR_NULL;
    const int64_t splits = static_splits(policy, param, max_seq_len);
    if (splits < 1) return HPCATTN_ERR_ARG;
    const int64_t rows = (int64_t)dims->batch * dims->num_kv_heads * splits;
    if (rows > INT32_MAX) return HPCATTN_ERR_SHAPE;
    if (part_o_rows < rows) return HPCATTN_ERR_WORKSPACE;
    DecodeParams p = make_params(dims, q, q_scale, k_pages, v_pages, k_scale, v_scale,
                                 page_table, part_o, part_lse);
    p.seq_lens = seq_lens;
    p.policy = policy;
    p.param = param;
    p.splits = (int32_t)splits;
    hipError_t e = launch_static_decode(p, dims->head_dim, dims->kv_dtype, (hipStream_t)stream);
    if (e != hipSuccess) return HPCATTN_ERR_LAUNCH;
    CombineParams c{};
    c.part_o = part_o;
    c.part_lse = part_lse;
    c.seg_off = nullptr;
    c.stride = (int32_t)splits;
    c.out = out;
    c.out_lse = out_lse;
    c.S = dims->batch * dims->num_kv_heads;
    c.G = p.G;
    c.D = dims->head_dim;
    c.R = dims->q_rows;
    c.Hkv = dims->num_kv_heads;
    return launch_status(launch_combine(c, (hipStream_t)stream));
}

int hpcattn_probe_stream_read(const void *buf, size_t bytes, int32_t workgroups, int32_t flags,
                              uint32_t *sink, void *stream) {
    if (!buf || !sink) return HPCATTN_ERR_NULL;
    if (bytes < 16 || bytes % 16 || workgroups < 1 || (flags & ~3)) return HPCATTN_ERR_ARG;
    if (flags & 2) {   // a power-of-two number of 16 KB chunks
        const size_t n = bytes / 16384;
        if (bytes % 16384 || n == 0 || (n & (n - 1))) return HPCATTN_ERR_ARG;
    }
    return launch_status(
        launch_stream_read(buf, bytes, workgroups, flags, sink, (hipStream_t)stream));
}

int hpcattn_prologue(const hpcattn_prologue_dims *d, const void *qkv, const int32_t *positions,
                     const int32_t *cache_slots, const float *q_norm_w, const float *k_norm_w,
                     void *q_out, float *q_scale, void *k_pages, void *v_pages, float *k_scale,
                     float *v_scale, void *stream) {
    if (!d) return HPCATTN_ERR_NULL;
    if (d->num_tokens < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
        (d->head_dim != 64 && d->head_dim != 128) || d->num_pages < 1 ||
        (int64_t)d->num_tokens * (d->num_q_heads + 2 * d->num_kv_heads) > INT32_MAX * 4ll)
        return HPCATTN_ERR_SHAPE;
    if (d->kv_dtype != HPCATTN_KV_BF16 && d->kv_dtype != HPCATTN_KV_FP8_E4M3)
        return HPCATTN_ERR_DTYPE;
    if ((d->flags & ~(HPCATTN_PROLOGUE_ROPE | HPCATTN_PROLOGUE_HADAMARD)) ||
        !(d->eps >= 0.f) || !std::isfinite(d->eps) || !(d->rope_base > 0.f) ||
        !std::isfinite(d->rope_base))
        return HPCATTN_ERR_ARG;
    if (!qkv || !cache_slots || !q_out || !k_pages || !v_pages) return HPCATTN_ERR_NULL;
    if ((d->flags & HPCATTN_PROLOGUE_ROPE) && !positions) return HPCATTN_ERR_NULL;
    const bool fp8 = d->kv_dtype == HPCATTN_KV_FP8_E4M3;
    if (fp8 ? !(q_scale && k_scale && v_scale) : (q_scale || k_scale || v_scale))
        return HPCATTN_ERR_DTYPE;
    PrologueParams p{};
    p.qkv = qkv;
    p.positions = positions;
    p.cache_slots = cache_slots;
    p.q_norm_w = q_norm_w;
    p.k_norm_w = k_norm_w;
    p.q_out = q_out;
    p.q_scale = q_scale;
    p.k_pages = k_pages;
    p.v_pages = v_pages;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.T = d->num_tokens;
    p.Hq = d->num_q_heads;
    p.Hkv = d->num_kv_heads;
    p.num_pages = d->num_pages;
    p.kv_dtype = d->kv_dtype;
    p.flags = d->flags;
    p.eps = d->eps;
    p.log2_base = std::log2((double)d->rope_base);
    return launch_status(launch_prologue(p, d->head_dim, (hipStream_t)stream));
}

const char *hpcattn_strerror(int status) {
    switch (status) {
    case HPCATTN_OK: return "ok";
    case HPCATTN_ERR_NULL: return "a required pointer is NULL";
    case HPCATTN_ERR_SHAPE: return "a size is out of range or inconsistent";
    case HPCATTN_ERR_DTYPE: return "unknown KV dtype, or scales given for bf16 / missing for fp8";
    case HPCATTN_ERR_WORKSPACE: return "a caller buffer is smaller than required";
    case HPCATTN_ERR_LAUNCH: return "the HIP runtime reported a launch error";
    case HPCATTN_ERR_ARG: return "an argument is out of range";
    default: return "unknown status";
    }
}

int hpcattn_version(void) { return 200; }

}  // extern "C"
