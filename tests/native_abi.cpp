// A decode step driven from C++ through include/hpcattn.h alone: device
// buffers from hipMalloc, no Python.  Checks that the C ABI is complete and
// usable as declared:
//   * plan -> decode -> combine, hpcattn_decode_combine and
//     hpcattn_decode_combine_noalloc on the same inputs agree with the fp64
//     oracle (oracle/liboracle.so, test infrastructure) at the bf16
//     tolerance (max |d| <= 2e-2, mean |d| <= 2e-3, |d lse| <= 2e-2);
//   * the fused call leaves its tickets at zero;
//   * a partial buffer declared too small is refused on the host
//     (HPCATTN_ERR_WORKSPACE) and nothing runs.
// Exit status 0 when every check holds; each failure is printed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "hpcattn.h"

extern "C" {
// The oracle's shape struct and attention (oracle/oracle.c).
typedef struct {
    int32_t batch, num_q_heads, num_kv_heads, head_dim, max_pages, num_pages, kv_fp8, q_rows;
    double sm_scale;
} orc_dims;
int orc_attention(const orc_dims *dm, const void *q, const float *q_scale, const void *k_pages,
                  const void *v_pages, const float *k_scale, const float *v_scale,
                  const int32_t *page_table, const int32_t *seq_lens, const int32_t *pairs,
                  int32_t n_pairs, double *out, double *out_lse);
}

namespace {

int failures = 0;

#define CHECK_HIP(x)                                                                    \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            std::printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__,     \
                        __LINE__);                                                      \
            return 1;                                                                   \
        }                                                                               \
    } while (0)

#define EXPECT(cond, ...)                                \
    do {                                                 \
        if (!(cond)) {                                   \
            std::printf("FAILED %s: ", #cond);           \
            std::printf(__VA_ARGS__);                    \
            std::printf("\n");                           \
            ++failures;                                  \
        }                                                \
    } while (0)

uint64_t lcg = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg >> 32);
}
float next_unit() { return (next_u32() >> 8) * (2.0f / 16777216.0f) - 1.0f; }   // [-1, 1)

uint16_t to_bf16(float f) {   // round to nearest even
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
float from_bf16(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

template <class T>
T *device_copy(const std::vector<T> &h) {
    T *d = nullptr;
    if (hipMalloc(&d, h.size() * sizeof(T)) != hipSuccess) return nullptr;
    if (hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess)
        return nullptr;
    return d;
}

// out (bf16) and out_lse against the oracle's fp64 values.
void compare(const char *what, const std::vector<uint16_t> &out, const std::vector<float> &lse,
             const std::vector<double> &ref_o, const std::vector<double> &ref_l, int D) {
    double max_abs = 0, sum_abs = 0, lse_max = 0;
    for (size_t i = 0; i < out.size(); ++i) {
        const double d = std::fabs((double)from_bf16(out[i]) - ref_o[i]);
        EXPECT(std::isfinite(d), "%s: element %zu not finite", what, i);
        max_abs = d > max_abs ? d : max_abs;
        sum_abs += d;
    }
    for (size_t r = 0; r < lse.size(); ++r) {
        if (std::isinf(ref_l[r])) {
            EXPECT(std::isinf(lse[r]) && lse[r] < 0, "%s: row %zu lse %g, want -inf", what, r,
                   (double)lse[r]);
            for (int e = 0; e < D; ++e)
                EXPECT(from_bf16(out[r * D + e]) == 0.f, "%s: empty row %zu not zero", what, r);
            continue;
        }
        const double d = std::fabs((double)lse[r] - ref_l[r]);
        lse_max = d > lse_max ? d : lse_max;
    }
    const double mean_abs = sum_abs / (double)out.size();
    std::printf("%s: max_abs %.3g mean_abs %.3g lse_max_abs %.3g\n", what, max_abs, mean_abs,
                lse_max);
    EXPECT(max_abs <= 2e-2, "%s: max_abs %g", what, max_abs);
    EXPECT(mean_abs <= 2e-3, "%s: mean_abs %g", what, mean_abs);
    EXPECT(lse_max <= 2e-2, "%s: lse_max_abs %g", what, lse_max);
}

}  // namespace

int main() {
    // Six requests of ragged lengths (an empty one included), 2 KV heads of
    // 8 query heads each, D = 128, bf16; 40 bins with a floor of 1 tile, so
    // long requests are cut into many chunks and the fused call fuses.
    const std::vector<int32_t> lens = {1, 63, 0, 65, 1000, 4100};
    const int B = (int)lens.size(), Hkv = 2, G = 8, Hq = Hkv * G, D = 128;
    const int P = 40, m = 1;
    int max_pages = 0, num_pages = 0;
    for (int L : lens) {
        const int n = (L + 63) / 64;
        max_pages = n > max_pages ? n : max_pages;
        num_pages += n;
    }
    num_pages += 3;   // spare pages no request uses

    // Pages handed out in order, then shuffled; unused table entries are -1.
    std::vector<int32_t> perm(num_pages);
    for (int i = 0; i < num_pages; ++i) perm[i] = i;
    for (int i = num_pages - 1; i > 0; --i) std::swap(perm[i], perm[next_u32() % (i + 1)]);
    std::vector<int32_t> table((size_t)B * max_pages, -1);
    for (int b = 0, next = 0; b < B; ++b)
        for (int t = 0; t < (lens[b] + 63) / 64; ++t) table[(size_t)b * max_pages + t] = perm[next++];

    std::vector<uint16_t> q((size_t)B * Hq * D), k((size_t)num_pages * Hkv * 64 * D),
        v(k.size());
    for (auto &x : q) x = to_bf16(next_unit());
    for (auto &x : k) x = to_bf16(next_unit());
    for (auto &x : v) x = to_bf16(next_unit());
    const float sm_scale = 1.0f / std::sqrt((float)D);

    // The oracle's answer.
    const orc_dims od{B, Hq, Hkv, D, max_pages, num_pages, 0, 1, (double)sm_scale};
    std::vector<double> ref_o((size_t)B * Hq * D), ref_l((size_t)B * Hq);
    if (orc_attention(&od, q.data(), nullptr, k.data(), v.data(), nullptr, nullptr, table.data(),
                      lens.data(), nullptr, 0, ref_o.data(), ref_l.data()) != 0) {
        std::printf("oracle failed\n");
        return 1;
    }

    // Device side.
    uint16_t *dq = device_copy(q), *dk = device_copy(k), *dv = device_copy(v);
    int32_t *dtable = device_copy(table), *dlens = device_copy(lens);
    if (!dq || !dk || !dv || !dtable || !dlens) {
        std::printf("device allocation failed\n");
        return 1;
    }
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));

    hpcattn_task_map map{};
    map.bytes = hpcattn_task_map_bytes(B, Hkv, P);
    CHECK_HIP(hipMalloc(&map.words, map.bytes));
    EXPECT(hpcattn_plan(dlens, B, Hkv, P, m, &map, stream) == HPCATTN_OK, "plan");

    const hpcattn_dims dims{B, Hq, Hkv, D, max_pages, num_pages, HPCATTN_KV_BF16, sm_scale, 1};
    const int64_t rows = hpcattn_max_partials(B, Hkv, P);
    float *part_o, *part_lse, *lse1, *lse2, *lse3;
    void *out1, *out2, *out3;
    int32_t *tickets;
    CHECK_HIP(hipMalloc(&part_o, (size_t)rows * G * D * sizeof(float)));
    CHECK_HIP(hipMalloc(&part_lse, (size_t)rows * G * sizeof(float)));
    const size_t out_bytes = (size_t)B * Hq * D * 2, lse_bytes = (size_t)B * Hq * 4;
    CHECK_HIP(hipMalloc(&out1, out_bytes));
    CHECK_HIP(hipMalloc(&out2, out_bytes));
    CHECK_HIP(hipMalloc(&out3, out_bytes));
    CHECK_HIP(hipMalloc(&lse1, lse_bytes));
    CHECK_HIP(hipMalloc(&lse2, lse_bytes));
    CHECK_HIP(hipMalloc(&lse3, lse_bytes));
    CHECK_HIP(hipMalloc(&tickets, (size_t)B * Hkv * sizeof(int32_t)));
    CHECK_HIP(hipMemset(tickets, 0, (size_t)B * Hkv * sizeof(int32_t)));

    // Refused on the host: a partial buffer one row short.
    EXPECT(hpcattn_decode(&dims, dq, nullptr, dk, dv, nullptr, nullptr, dtable, &map, part_o,
                          part_lse, rows - 1, stream) == HPCATTN_ERR_WORKSPACE,
           "short partial buffer");

    EXPECT(hpcattn_decode(&dims, dq, nullptr, dk, dv, nullptr, nullptr, dtable, &map, part_o,
                          part_lse, rows, stream) == HPCATTN_OK,
           "decode");
    EXPECT(hpcattn_combine(&dims, &map, part_o, part_lse, out1, lse1, stream) == HPCATTN_OK,
           "combine");
    EXPECT(hpcattn_decode_combine(&dims, dq, nullptr, dk, dv, nullptr, nullptr, dtable, &map,
                                  part_o, part_lse, rows, tickets, (int64_t)B * Hkv, out2, lse2,
                                  stream) == HPCATTN_OK,
           "decode_combine");
    EXPECT(hpcattn_decode_combine_noalloc(&dims, dq, nullptr, dk, dv, nullptr, nullptr, dtable,
                                          &map, out3, lse3, stream) == HPCATTN_OK,
           "decode_combine_noalloc");
    CHECK_HIP(hipStreamSynchronize(stream));

    std::vector<int32_t> header(8), tk((size_t)B * Hkv);
    CHECK_HIP(hipMemcpy(header.data(), map.words, 32, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(tk.data(), tickets, tk.size() * 4, hipMemcpyDeviceToHost));
    std::printf("plan: T %d tiles, %d bins used, %d descriptors, error word %d\n", header[0],
                header[1], header[4], header[7]);
    EXPECT(header[7] == 0, "plan error word %d", header[7]);
    EXPECT(header[4] > B * Hkv, "descriptors %d: some segment must be cut", header[4]);
    for (size_t i = 0; i < tk.size(); ++i) EXPECT(tk[i] == 0, "ticket %zu = %d", i, tk[i]);

    const struct {
        const char *what;
        void *out;
        float *lse;
    } runs[] = {{"decode + combine", out1, lse1},
                {"decode_combine", out2, lse2},
                {"decode_combine_noalloc", out3, lse3}};
    for (const auto &r : runs) {
        std::vector<uint16_t> o((size_t)B * Hq * D);
        std::vector<float> l((size_t)B * Hq);
        CHECK_HIP(hipMemcpy(o.data(), r.out, out_bytes, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(l.data(), r.lse, lse_bytes, hipMemcpyDeviceToHost));
        compare(r.what, o, l, ref_o, ref_l, D);
    }

    CHECK_HIP(hipFree(dq));
    CHECK_HIP(hipFree(dk));
    CHECK_HIP(hipFree(dv));
    CHECK_HIP(hipFree(dtable));
    CHECK_HIP(hipFree(dlens));
    CHECK_HIP(hipFree(map.words));
    CHECK_HIP(hipFree(part_o));
    CHECK_HIP(hipFree(part_lse));
    CHECK_HIP(hipFree(out1));
    CHECK_HIP(hipFree(out2));
    CHECK_HIP(hipFree(out3));
    CHECK_HIP(hipFree(lse1));
    CHECK_HIP(hipFree(lse2));
    CHECK_HIP(hipFree(lse3));
    CHECK_HIP(hipFree(tickets));
    CHECK_HIP(hipStreamDestroy(stream));
    std::printf(failures ? "%d check(s) failed\n" : "all checks passed\n", failures);
    return failures ? 1 : 0;
}
