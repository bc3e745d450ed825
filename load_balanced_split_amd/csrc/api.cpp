// C ABI of libhpcattn: the launches.  Every entry point first runs its
// host-side checks (validate.cpp), before anything is enqueued, so a
// rejected call has no side effect.  See hpcattn.h for the contract of each
// entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "common.h"
#include "hpcattn.h"
#include "validate.h"

using namespace hpcattn;

namespace {

constexpr float kLog2e = 1.4426950408889634f;

int launch_status(hipError_t e) { return e == hipSuccess ? HPCATTN_OK : HPCATTN_ERR_LAUNCH; }

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

}  // namespace

extern "C" {

int hpcattn_plan(const int32_t *seq_lens, int32_t batch, int32_t num_kv_heads,
                 int32_t num_bins, int32_t min_tiles, hpcattn_task_map *map, void *stream) {
    const int rc = check_plan(seq_lens, batch, num_kv_heads, num_bins, min_tiles, map);
    if (rc) return rc;
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
    const int rc = check_decode(dims, q, q_scale, k_pages, v_pages, k_scale, v_scale, page_table,
                                map, part_o, part_lse, part_o_rows);
    if (rc) return rc;
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
    const int rc = check_decode_combine(dims, q, q_scale, k_pages, v_pages, k_scale, v_scale,
                                        page_table, map, part_o, part_lse, part_o_rows, tickets,
                                        num_tickets, out);
    if (rc) return rc;
    DecodeParams p = make_params(dims, q, q_scale, k_pages, v_pages, k_scale, v_scale,
                                 page_table, part_o, part_lse);
    p.map = map->words;
    p.P = map->num_bins;
    const int32_t rows = dims->q_rows * (dims->num_q_heads / dims->num_kv_heads);
    if (!fuse_combine(dims, map) ||
        !fused_keeps_residency(dims->head_dim, dims->kv_dtype, rows)) {
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
    const int rc = check_combine(dims, map, part_o, part_lse, out);
    if (rc) return rc;
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

int hpcattn_static_decode(const hpcattn_dims *dims, int32_t policy, int32_t param,
                          int32_t max_seq_len, const int32_t *seq_lens, const void *q,
                          const float *q_scale, const void *k_pages, const void *v_pages,
                          const float *k_scale, const float *v_scale,
                          const int32_t *page_table, float *part_o, float *part_lse,
                          int64_t part_o_rows, void *out, float *out_lse, void *stream) {
    const int rc = check_static(dims, policy, param, max_seq_len, seq_lens, q, q_scale, k_pages,
                                v_pages, k_scale, v_scale, page_table, part_o, part_lse,
                                part_o_rows, out);
    if (rc) return rc;
    const int64_t splits = static_splits(policy, param, max_seq_len);
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
    const int rc = check_probe(buf, bytes, workgroups, flags, sink);
    if (rc) return rc;
    return launch_status(
        launch_stream_read(buf, bytes, workgroups, flags, sink, (hipStream_t)stream));
}

int hpcattn_prologue(const hpcattn_prologue_dims *d, const void *qkv, const int32_t *positions,
                     const int32_t *cache_slots, const float *q_norm_w, const float *k_norm_w,
                     void *q_out, float *q_scale, void *k_pages, void *v_pages, float *k_scale,
                     float *v_scale, void *stream) {
    const int rc = check_prologue(d, qkv, positions, cache_slots, q_out, q_scale, k_pages,
                                  v_pages, k_scale, v_scale);
    if (rc) return rc;
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
    for (int i = 0; i < d->head_dim / 2; ++i)
        p.freq[i] = std::pow((double)d->rope_base, -2.0 * i / d->head_dim);
    return launch_status(launch_prologue(p, d->head_dim, (hipStream_t)stream));
}

}  // extern "C"
