// Host-side argument validation of the C ABI.  Plain C++ with no HIP
// dependency, so that it also builds with g++ on its own and runs under the
// host address and undefined-behaviour sanitizers.  Each check returns
// HPCATTN_OK or the status the entry point returns, and touches no device
// memory: the pointers are only compared with NULL.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "hpcattn.h"

namespace hpcattn {

// B in [1, HPCATTN_MAX_BATCH], H_kv >= 1, P >= 1 and B H_kv + P - 1 partial
// slots addressable with int32.
bool sizes_ok(int32_t batch, int32_t num_kv_heads, int32_t num_bins);

// Partial slots per (request, KV head) of a static policy, or -1.
int64_t static_splits(int32_t policy, int32_t param, int32_t max_seq_len);

int check_dims(const hpcattn_dims *d);
int check_operands(const hpcattn_dims *d, const void *q, const float *q_scale,
                   const void *k_pages, const void *v_pages, const float *k_scale,
                   const float *v_scale, const int32_t *page_table);
int check_map(const hpcattn_dims *d, const hpcattn_task_map *map);

int check_plan(const int32_t *seq_lens, int32_t batch, int32_t num_kv_heads, int32_t num_bins,
               int32_t min_tiles, const hpcattn_task_map *map);
int check_decode(const hpcattn_dims *d, const void *q, const float *q_scale,
                 const void *k_pages, const void *v_pages, const float *k_scale,
                 const float *v_scale, const int32_t *page_table, const hpcattn_task_map *map,
                 const float *part_o, const float *part_lse, int64_t part_o_rows);
int check_decode_combine(const hpcattn_dims *d, const void *q, const float *q_scale,
                         const void *k_pages, const void *v_pages, const float *k_scale,
                         const float *v_scale, const int32_t *page_table,
                         const hpcattn_task_map *map, const float *part_o, const float *part_lse,
                         int64_t part_o_rows, const int32_t *tickets, int64_t num_tickets,
                         const void *out);
int check_combine(const hpcattn_dims *d, const hpcattn_task_map *map, const float *part_o,
                  const float *part_lse, const void *out);
int check_static(const hpcattn_dims *d, int32_t policy, int32_t param, int32_t max_seq_len,
                 const int32_t *seq_lens, const void *q, const float *q_scale,
                 const void *k_pages, const void *v_pages, const float *k_scale,
                 const float *v_scale, const int32_t *page_table, const float *part_o,
                 const float *part_lse, int64_t part_o_rows, const void *out);
int check_probe(const void *buf, size_t bytes, int32_t workgroups, int32_t flags,
                const uint32_t *sink);
int check_prologue(const hpcattn_prologue_dims *d, const void *qkv, const int32_t *positions,
                   const int32_t *cache_slots, const void *q_out, const float *q_scale,
                   const void *k_pages, const void *v_pages, const float *k_scale,
                   const float *v_scale);

// Whether decode + combine runs as one fused launch for this shape (else
// as decode, then combine).
bool fuse_combine(const hpcattn_dims *d, const hpcattn_task_map *map);

// Byte offsets of the allocation-free entry point's buffers inside its
// fixed scratch array: the tickets always at 0, HPCATTN_NOALLOC_MAX_SEGMENTS
// int32 (fixed, so that one call's partials never lie where a later call's
// tickets are expected to be zero); part_lse [rows, R G] fp32 at `lse`;
// part_o [rows, R G, D] fp32 at `o`, 256-byte aligned; `end` is the bytes used.
struct ScratchPlan {
    int64_t num_tickets, rows;
    int64_t lse, o, end;
};
ScratchPlan scratch_plan(const hpcattn_dims *d, const hpcattn_task_map *map);

// The checks of hpcattn_decode_combine_noalloc: those of decode_combine for
// the buffers the caller passes, then HPCATTN_ERR_WORKSPACE when the batch
// has more segments than tickets or the partials need more than the array.
int check_decode_combine_noalloc(const hpcattn_dims *d, const void *q, const float *q_scale,
                                 const void *k_pages, const void *v_pages, const float *k_scale,
                                 const float *v_scale, const int32_t *page_table,
                                 const hpcattn_task_map *map, const void *out);

}  // namespace hpcattn
