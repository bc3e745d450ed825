// Internal declarations shared by the HIP translation units of libhpcattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hpcattn.h"
#include "layout.h"

namespace hpcattn {

constexpr int kTile = HPCATTN_PAGE_SIZE;  // tokens per tile and per page
constexpr int kWaves = 4;                 // waves per decode workgroup
constexpr int kDecodeThreads = 64 * kWaves;
constexpr int kPlanThreads = 1024;

// Arguments of the decode kernels (dynamic and static), passed by value.
struct DecodeParams {
    const void *q;
    const float *q_scale;
    const void *k;
    const void *v;
    const float *k_scale;
    const float *v_scale;
    const int32_t *page_table;
    float *part_o;
    float *part_lse;
    // dynamic: task map; static: seq_lens
    const int32_t *map;
    const int32_t *seq_lens;
    int32_t B, Hq, Hkv, G, max_pages, num_pages;
    int32_t R;              // query rows per request (1 + draft tokens)
    int32_t P;              // bins (dynamic)
    int32_t policy, param;  // static split policy and its parameter
    int32_t splits;         // static: slots per segment
    float scale_log2;       // sm_scale * log2(e)
    // decode + combine in one launch (dynamic only; out == NULL: off)
    void *out;              // bf16 [B, R, Hq, D]
    float *out_lse;         // [B, R, Hq] or NULL
    int32_t *tickets;       // [B * Hkv], zero on entry and on exit
};

struct CombineParams {
    const float *part_o;
    const float *part_lse;
    const int32_t *seg_off;  // CSR of partial slots per segment, or NULL
    int32_t stride;          // when seg_off is NULL: segment s owns slots
                             // [s * stride, (s + 1) * stride)
    void *out;
    float *out_lse;
    int32_t S, G, D;
    int32_t R, Hkv;          // query rows per request; segment s = b * Hkv + h
    int64_t max_chunks;      // with seg_off: partial slots of the map (S + P - 1)
};

// Arguments of the prologue kernel.
struct PrologueParams {
    const void *qkv;
    const int32_t *positions;
    const int32_t *cache_slots;
    const float *q_norm_w;
    const float *k_norm_w;
    void *q_out;
    float *q_scale;
    void *k_pages;
    void *v_pages;
    float *k_scale;
    float *v_scale;
    int32_t T, Hq, Hkv, num_pages, kv_dtype, flags;
    float eps;
    double freq[64];            // RoPE frequencies base^(-2i/D), i < D/2
};

hipError_t launch_plan(const int32_t *seq_lens, int32_t B, int32_t Hkv, int32_t P,
                       int32_t m, int32_t *map, hipStream_t stream);
hipError_t launch_decode(const DecodeParams &p, int32_t head_dim, int32_t kv_dtype,
                         hipStream_t stream);
hipError_t launch_static_decode(const DecodeParams &p, int32_t head_dim, int32_t kv_dtype,
                                hipStream_t stream);
hipError_t launch_combine(const CombineParams &p, hipStream_t stream);
hipError_t launch_prologue(const PrologueParams &p, int32_t head_dim, hipStream_t stream);
// rows = R * G, the query rows that share one KV head's tiles.
int32_t decode_resident_per_cu(int32_t head_dim, int32_t kv_dtype, int32_t rows);
// Whether the fused decode + combine instance for this shape holds as many
// workgroups per CU as the decode alone (whose count sets the default bins).
bool fused_keeps_residency(int32_t head_dim, int32_t kv_dtype, int32_t rows);
hipError_t launch_stream_read(const void *buf, size_t bytes, int32_t workgroups, int32_t flags,
                              uint32_t *sink, hipStream_t stream);

}  // namespace hpcattn
