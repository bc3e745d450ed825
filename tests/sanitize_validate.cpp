// Host driver of the C ABI's argument validation (csrc/validate.cpp), built
// with g++ and the address and undefined-behaviour sanitizers by
// tests/test_sanitizers.py.  Every check runs on fake non-NULL pointers that
// are never dereferenced, over valid arguments and over the edges of every
// range, including the int32 limits where a product could wrap.  A signed
// overflow, an out-of-bounds access or a wrong status ends the run non-zero.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <limits>

#include "hpcattn.h"
#include "validate.h"

using namespace hpcattn;

static int failures = 0;

#define EXPECT(expr, want)                                                                 \
    do {                                                                                   \
        const long long got_ = (long long)(expr);                                          \
        if (got_ != (long long)(want)) {                                                   \
            fprintf(stderr, "%s:%d: %s = %lld, want %lld\n", __FILE__, __LINE__, #expr, got_, \
                    (long long)(want));                                                    \
            ++failures;                                                                    \
        }                                                                                  \
    } while (0)

static void *const F = (void *)0x10000;   // a fake device address
static const float *const FF = (const float *)0x10000;
static const int32_t *const FI = (const int32_t *)0x10000;
static const int32_t I32MAX = std::numeric_limits<int32_t>::max();
static const int32_t I32MIN = std::numeric_limits<int32_t>::min();

static hpcattn_dims dims(int32_t B = 4, int32_t Hq = 4, int32_t Hkv = 1, int32_t D = 64,
                         int32_t R = 1, int32_t dtype = HPCATTN_KV_BF16) {
    hpcattn_dims d{};
    d.batch = B;
    d.num_q_heads = Hq;
    d.num_kv_heads = Hkv;
    d.head_dim = D;
    d.max_pages_per_req = 16;
    d.num_pages = 22;
    d.kv_dtype = dtype;
    d.sm_scale = 0.125f;
    d.q_rows = R;
    return d;
}

static hpcattn_task_map map_for(int32_t B, int32_t Hkv, int32_t P, size_t bytes = 0) {
    hpcattn_task_map m{};
    m.words = (int32_t *)F;
    m.bytes = bytes ? bytes : hpcattn_task_map_bytes(B, Hkv, P);
    m.batch = B;
    m.num_kv_heads = Hkv;
    m.num_bins = P;
    m.min_tiles = 1;
    return m;
}

static void test_dims() {
    hpcattn_dims d = dims();
    EXPECT(check_dims(&d), HPCATTN_OK);
    EXPECT(check_dims(nullptr), HPCATTN_ERR_NULL);
    // q_rows * G must not wrap: 2^28 + 1 rows of 16 heads
    d = dims(4, 16, 1, 64, (1 << 28) + 1);
    EXPECT(check_dims(&d), HPCATTN_ERR_SHAPE);
    d = dims(4, 16, 1, 64, I32MAX);
    EXPECT(check_dims(&d), HPCATTN_ERR_SHAPE);
    d = dims(4, 16, 1, 64, I32MIN);
    EXPECT(check_dims(&d), HPCATTN_ERR_SHAPE);
    d = dims(4, 16, 1, 64, 4);   // 64 rows: the limit
    EXPECT(check_dims(&d), HPCATTN_OK);
    d = dims(4, 16, 1, 64, 5);
    EXPECT(check_dims(&d), HPCATTN_ERR_SHAPE);
    d = dims(I32MAX);
    EXPECT(check_dims(&d), HPCATTN_ERR_SHAPE);
    d = dims(I32MIN);
    EXPECT(check_dims(&d), HPCATTN_ERR_SHAPE);
    d = dims(4, I32MAX, I32MAX);   // G = 1 with 2^31 - 1 heads: a valid shape
    EXPECT(check_dims(&d), HPCATTN_OK);
    d = dims(4, I32MIN, I32MIN);
    EXPECT(check_dims(&d), HPCATTN_ERR_SHAPE);
    d = dims(4, 4, 0);
    EXPECT(check_dims(&d), HPCATTN_ERR_SHAPE);
    d = dims(4, 6, 4);
    EXPECT(check_dims(&d), HPCATTN_ERR_SHAPE);
    d = dims(4, 34, 2);
    EXPECT(check_dims(&d), HPCATTN_ERR_SHAPE);
    d = dims(4, 4, 1, 96);
    EXPECT(check_dims(&d), HPCATTN_ERR_SHAPE);
    d = dims(4, 4, 1, 64, 1, 7);
    EXPECT(check_dims(&d), HPCATTN_ERR_DTYPE);
    d = dims();
    d.sm_scale = std::numeric_limits<float>::infinity();
    EXPECT(check_dims(&d), HPCATTN_ERR_ARG);
    d.sm_scale = std::numeric_limits<float>::quiet_NaN();
    EXPECT(check_dims(&d), HPCATTN_ERR_ARG);
}

static void test_map_and_plan() {
    hpcattn_dims d = dims();
    hpcattn_task_map m = map_for(4, 1, 8);
    EXPECT(check_map(&d, &m), HPCATTN_OK);
    EXPECT(check_map(&d, nullptr), HPCATTN_ERR_NULL);
    hpcattn_task_map small = map_for(4, 1, 8, 16);
    EXPECT(check_map(&d, &small), HPCATTN_ERR_WORKSPACE);
    hpcattn_task_map wide = map_for(4, 1, I32MAX);   // B H_kv + P - 1 > INT32_MAX
    EXPECT(check_map(&d, &wide), HPCATTN_ERR_SHAPE);
    EXPECT(sizes_ok(HPCATTN_MAX_BATCH, I32MAX, 1), false);
    EXPECT(sizes_ok(1, 1, I32MAX), true);
    EXPECT(sizes_ok(2, 1, I32MAX), false);
    EXPECT(check_plan(FI, 4, 1, 8, 2, &m), HPCATTN_OK);
    EXPECT(check_plan(nullptr, 4, 1, 8, 2, &m), HPCATTN_ERR_NULL);
    EXPECT(check_plan(FI, 4, 1, 8, 0, &m), HPCATTN_ERR_ARG);
    EXPECT(check_plan(FI, 4, 1, 8, I32MIN, &m), HPCATTN_ERR_ARG);
    EXPECT(check_plan(FI, HPCATTN_MAX_BATCH + 1, 1, 8, 2, &m), HPCATTN_ERR_SHAPE);
    EXPECT(check_plan(FI, 4, I32MAX, I32MAX, 2, &m), HPCATTN_ERR_SHAPE);
    EXPECT(check_plan(FI, 4, 1, 8, 2, &small), HPCATTN_ERR_WORKSPACE);
    // the size queries at the int32 limits
    EXPECT(hpcattn_task_map_bytes(HPCATTN_MAX_BATCH, I32MAX, I32MAX) > 0, true);
    EXPECT(hpcattn_max_partials(I32MAX, I32MAX, I32MAX) > 0, true);
    EXPECT(hpcattn_max_partials(0, 1, 1), 0);
    EXPECT(hpcattn_task_map_bytes(1, 1, I32MIN), 0);
}

static void test_decode_paths() {
    hpcattn_dims d = dims();
    hpcattn_task_map m = map_for(4, 1, 8);
    const int64_t rows = hpcattn_max_partials(4, 1, 8);
    float *po = (float *)F;
    EXPECT(check_decode(&d, F, nullptr, F, F, nullptr, nullptr, FI, &m, po, po, rows), HPCATTN_OK);
    EXPECT(check_decode(&d, F, nullptr, F, F, nullptr, nullptr, FI, &m, po, po, rows - 1),
           HPCATTN_ERR_WORKSPACE);
    EXPECT(check_decode(&d, F, FF, F, F, nullptr, nullptr, FI, &m, po, po, rows),
           HPCATTN_ERR_DTYPE);
    hpcattn_dims d8 = dims(4, 4, 1, 64, 1, HPCATTN_KV_FP8_E4M3);
    EXPECT(check_decode(&d8, F, FF, F, F, FF, FF, FI, &m, po, po, rows), HPCATTN_OK);
    EXPECT(check_decode(&d8, F, FF, F, F, FF, nullptr, FI, &m, po, po, rows), HPCATTN_ERR_DTYPE);
    hpcattn_dims wrap = dims(4, 16, 1, 64, (1 << 28) + 1);
    EXPECT(check_decode(&wrap, F, nullptr, F, F, nullptr, nullptr, FI, &m, po, po, rows),
           HPCATTN_ERR_SHAPE);
    EXPECT(check_decode_combine(&d, F, nullptr, F, F, nullptr, nullptr, FI, &m, po, po, rows,
                                FI, 4, F),
           HPCATTN_OK);
    EXPECT(check_decode_combine(&d, F, nullptr, F, F, nullptr, nullptr, FI, &m, po, po, rows,
                                FI, 3, F),
           HPCATTN_ERR_WORKSPACE);
    EXPECT(check_decode_combine(&d, F, nullptr, F, F, nullptr, nullptr, FI, &m, po, po, rows,
                                nullptr, 4, F),
           HPCATTN_ERR_NULL);
    EXPECT(check_combine(&d, &m, po, po, F), HPCATTN_OK);
    EXPECT(check_combine(&d, &m, po, po, nullptr), HPCATTN_ERR_NULL);
    EXPECT(fuse_combine(&d, &m), true);
    hpcattn_dims rows48 = dims(4, 8, 1, 128, 6);
    EXPECT(fuse_combine(&rows48, &m), true);   // a mean of 3 chunks
    hpcattn_task_map m5 = map_for(4, 1, 16);   // a mean of 5 chunks
    EXPECT(fuse_combine(&d, &m5), true);
    EXPECT(fuse_combine(&rows48, &m5), false);
    hpcattn_task_map many = map_for(1, 1, I32MAX);   // mean chunks far above 8
    hpcattn_dims d1 = dims(1);
    EXPECT(fuse_combine(&d1, &many), false);
}

static void test_noalloc() {
    hpcattn_dims d = dims();
    hpcattn_task_map m = map_for(4, 1, 8);
    EXPECT(check_decode_combine_noalloc(&d, F, nullptr, F, F, nullptr, nullptr, FI, &m, F),
           HPCATTN_OK);
    EXPECT(check_decode_combine_noalloc(&d, F, nullptr, F, F, nullptr, nullptr, FI, &m, nullptr),
           HPCATTN_ERR_NULL);
    const ScratchPlan s = scratch_plan(&d, &m);
    EXPECT(s.lse, 4 * HPCATTN_NOALLOC_MAX_SEGMENTS);   // tickets first, at a fixed size
    EXPECT(s.o % 256, 0);
    EXPECT(s.end, s.o + 4 * s.rows * 4 * 64);
    // 8192 x 2 segments of 8 rows at D = 128: partials past the array
    hpcattn_dims big = dims(HPCATTN_MAX_BATCH, 16, 2, 128);
    hpcattn_task_map mb = map_for(HPCATTN_MAX_BATCH, 2, 512);
    EXPECT(check_decode_combine_noalloc(&big, F, nullptr, F, F, nullptr, nullptr, FI, &mb, F),
           HPCATTN_ERR_WORKSPACE);
    // more segments than tickets, however small the partials
    hpcattn_dims wide = dims(HPCATTN_MAX_BATCH, 9, 9, 64);
    hpcattn_task_map mw = map_for(HPCATTN_MAX_BATCH, 9, 1);
    EXPECT(check_decode_combine_noalloc(&wide, F, nullptr, F, F, nullptr, nullptr, FI, &mw, F),
           HPCATTN_ERR_WORKSPACE);
    // the largest map the checks admit: no overflow in the plan's products
    hpcattn_dims huge = dims(HPCATTN_MAX_BATCH, 16, 1, 128, 4);
    hpcattn_task_map mh = map_for(HPCATTN_MAX_BATCH, 1, I32MAX - HPCATTN_MAX_BATCH + 1);
    EXPECT(check_decode_combine_noalloc(&huge, F, nullptr, F, F, nullptr, nullptr, FI, &mh, F),
           HPCATTN_ERR_WORKSPACE);
}

static void test_static() {
    hpcattn_dims d = dims();
    float *po = (float *)F;
    EXPECT(check_static(&d, 0, 8, 1000, FI, F, nullptr, F, F, nullptr, nullptr, FI, po, po, 32,
                        F),
           HPCATTN_OK);
    EXPECT(check_static(&d, 0, 8, 1000, FI, F, nullptr, F, F, nullptr, nullptr, FI, po, po, 31,
                        F),
           HPCATTN_ERR_WORKSPACE);
    EXPECT(check_static(&d, 2, 8, 1000, FI, F, nullptr, F, F, nullptr, nullptr, FI, po, po, 32,
                        F),
           HPCATTN_ERR_ARG);
    EXPECT(check_static(&d, 1, 100, 1000, FI, F, nullptr, F, F, nullptr, nullptr, FI, po, po,
                        32, F),
           HPCATTN_ERR_ARG);
    EXPECT(check_static(&d, 1, 256, -1, FI, F, nullptr, F, F, nullptr, nullptr, FI, po, po, 32,
                        F),
           HPCATTN_ERR_ARG);
    // B H_kv splits beyond int32 (and beyond int64 when multiplied out)
    hpcattn_dims big = dims(HPCATTN_MAX_BATCH, I32MAX, I32MAX);
    EXPECT(check_static(&big, 0, I32MAX, 1000, FI, F, nullptr, F, F, nullptr, nullptr, FI, po,
                        po, INT64_MAX, F),
           HPCATTN_ERR_SHAPE);
    EXPECT(check_static(&d, 1, 64, I32MAX, FI, F, nullptr, F, F, nullptr, nullptr, FI, po, po,
                        INT64_MAX, F),
           HPCATTN_OK);   // 4 x 2^25 chunks of one page: within int32
    EXPECT(hpcattn_static_max_partials(HPCATTN_MAX_BATCH, I32MAX, 0, I32MAX, 1000), 0);
    EXPECT(hpcattn_static_max_partials(4, 2, 0, 8, 1000), 64);
    EXPECT(hpcattn_static_max_partials(4, 2, 1, 256, 1000), 32);
    EXPECT(hpcattn_static_max_partials(4, 2, 1, 64, I32MAX), 8 * ((int64_t)I32MAX / 64 + 1));
    EXPECT(hpcattn_static_max_partials(64, 2, 1, 64, I32MAX), 0);
    EXPECT(static_splits(1, 64, I32MAX), (int64_t)I32MAX / 64 + 1);
    EXPECT(static_splits(1, 64, 0), 1);
    EXPECT(static_splits(0, I32MIN, 10), -1);
}

static void test_probe_and_prologue() {
    const uint32_t *sink = (const uint32_t *)F;
    EXPECT(check_probe(F, 1024, 8, 0, sink), HPCATTN_OK);
    EXPECT(check_probe(F, 1000, 8, 0, sink), HPCATTN_ERR_ARG);
    EXPECT(check_probe(F, 3 * 16384, 8, 2, sink), HPCATTN_ERR_ARG);
    EXPECT(check_probe(F, 4 * 16384, 8, 3, sink), HPCATTN_OK);
    EXPECT(check_probe(F, SIZE_MAX - 15, 8, 0, sink), HPCATTN_OK);
    EXPECT(check_probe(F, 1024, I32MIN, 0, sink), HPCATTN_ERR_ARG);
    hpcattn_prologue_dims p{};
    p.num_tokens = 4;
    p.num_q_heads = 8;
    p.num_kv_heads = 2;
    p.head_dim = 128;
    p.num_pages = 4;
    p.kv_dtype = HPCATTN_KV_BF16;
    p.flags = HPCATTN_PROLOGUE_ROPE;
    p.eps = 1e-6f;
    p.rope_base = 10000.f;
    EXPECT(check_prologue(&p, F, FI, FI, F, nullptr, F, F, nullptr, nullptr), HPCATTN_OK);
    EXPECT(check_prologue(&p, F, nullptr, FI, F, nullptr, F, F, nullptr, nullptr),
           HPCATTN_ERR_NULL);
    {   // no tokens: nothing is touched, NULL buffers are fine (the other checks still hold)
        hpcattn_prologue_dims z = p;
        z.num_tokens = 0;
        EXPECT(check_prologue(&z, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr, nullptr), HPCATTN_OK);
        z.head_dim = 96;
        EXPECT(check_prologue(&z, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr, nullptr), HPCATTN_ERR_SHAPE);
    }
    hpcattn_prologue_dims q = p;   // H_q + 2 H_kv must not wrap in int32
    q.num_q_heads = I32MAX;
    q.num_kv_heads = I32MAX;
    EXPECT(check_prologue(&q, F, FI, FI, F, nullptr, F, F, nullptr, nullptr), HPCATTN_ERR_SHAPE);
    q = p;   // 12 heads: one wave per token, T * 64 work-items below 2^32
    q.num_tokens = I32MAX;
    EXPECT(check_prologue(&q, F, FI, FI, F, nullptr, F, F, nullptr, nullptr), HPCATTN_ERR_SHAPE);
    q.num_tokens = 1 << 26;
    EXPECT(check_prologue(&q, F, FI, FI, F, nullptr, F, F, nullptr, nullptr), HPCATTN_ERR_SHAPE);
    q.num_tokens = (1 << 26) - 1;
    EXPECT(check_prologue(&q, F, FI, FI, F, nullptr, F, F, nullptr, nullptr), HPCATTN_OK);
    q.num_tokens = 4;
    q.num_q_heads = HPCATTN_PROLOGUE_MAX_HEADS - 4;   // heads = the maximum
    EXPECT(check_prologue(&q, F, FI, FI, F, nullptr, F, F, nullptr, nullptr), HPCATTN_OK);
    q.num_q_heads += 1;
    EXPECT(check_prologue(&q, F, FI, FI, F, nullptr, F, F, nullptr, nullptr), HPCATTN_ERR_SHAPE);
    q = p;
    q.eps = std::numeric_limits<float>::quiet_NaN();
    EXPECT(check_prologue(&q, F, FI, FI, F, nullptr, F, F, nullptr, nullptr), HPCATTN_ERR_ARG);
    q = p;
    q.flags = 1 << 30;
    EXPECT(check_prologue(&q, F, FI, FI, F, nullptr, F, F, nullptr, nullptr), HPCATTN_ERR_ARG);
    q = p;
    q.kv_dtype = HPCATTN_KV_FP8_E4M3;
    EXPECT(check_prologue(&q, F, FI, FI, F, nullptr, F, F, nullptr, nullptr), HPCATTN_ERR_DTYPE);
    EXPECT(check_prologue(&q, F, FI, FI, F, FF, F, F, FF, FF), HPCATTN_OK);
}

int main() {
    test_dims();
    test_map_and_plan();
    test_decode_paths();
    test_static();
    test_noalloc();
    test_probe_and_prologue();
    for (int s = -8; s <= 1; ++s)
        if (!hpcattn_strerror(s)) ++failures;
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("validation: all checks passed\n");
    return 0;
}
