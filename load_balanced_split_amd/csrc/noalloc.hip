// hpcattn_decode_combine_noalloc: decode + combine in one call that
// allocates nothing, for callers that cannot call hipMalloc (code under HIP
// graph capture, serving loops that forbid it).  Its partials and tickets
// live in `scratch` below, one array per device, which the loader places in
// device memory with the library's code and which stays until the process
// ends.
//
// In host code `scratch` names a host-side stand-in, not the device array:
// a kernel handed that name would access an address that is not mapped on
// the GPU.  So its device address is taken once per device, with that
// device current, by hipGetSymbolAddress, and only that address is used.
#include <mutex>

#include "common.h"
#include "validate.h"

namespace hpcattn {
namespace {

__device__ __align__(256) static unsigned char scratch[HPCATTN_NOALLOC_SCRATCH_BYTES];

// Zero the ticket block (n int32 at t), by a kernel rather than a memset
// node, so that a call captured in a graph stays correct on every replay.
__global__ void __launch_bounds__(256) clear_tickets(int32_t *t, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) t[i] = 0;
}

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    std::once_flag once;
    unsigned char *ptr = nullptr;   // the device address of `scratch`
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// The current device's scratch address; on its first call for a device it
// looks the address up and enqueues the clearing of the tickets on `stream`.
int scratch_of_current_device(hipStream_t stream, unsigned char **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return HPCATTN_ERR_LAUNCH;
    DeviceScratch &s = g_scratch[dev];
    std::call_once(s.once, [&] {
        void *p = nullptr;
        s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (s.err != hipSuccess) return;
        s.ptr = static_cast<unsigned char *>(p);
        hipLaunchKernelGGL(clear_tickets, dim3(64), dim3(256), 0, stream,
                           reinterpret_cast<int32_t *>(s.ptr), HPCATTN_NOALLOC_MAX_SEGMENTS);
        s.err = hipGetLastError();
    });
    if (s.err != hipSuccess || !s.ptr) return HPCATTN_ERR_LAUNCH;
    *out = s.ptr;
    return HPCATTN_OK;
}

}  // namespace
}  // namespace hpcattn

using namespace hpcattn;

extern "C" int hpcattn_decode_combine_noalloc(const hpcattn_dims *dims, const void *q,
                                              const float *q_scale, const void *k_pages,
                                              const void *v_pages, const float *k_scale,
                                              const float *v_scale, const int32_t *page_table,
                                              const hpcattn_task_map *map, void *out,
                                              float *out_lse, void *stream) {
    int rc = check_decode_combine_noalloc(dims, q, q_scale, k_pages, v_pages, k_scale, v_scale,
                                          page_table, map, out);
    if (rc) return rc;
    unsigned char *base = nullptr;
    rc = scratch_of_current_device((hipStream_t)stream, &base);
    if (rc) return rc;
    const ScratchPlan s = scratch_plan(dims, map);
    return hpcattn_decode_combine(dims, q, q_scale, k_pages, v_pages, k_scale, v_scale,
                                  page_table, map, reinterpret_cast<float *>(base + s.o),
                                  reinterpret_cast<float *>(base + s.lse), s.rows,
                                  reinterpret_cast<int32_t *>(base), s.num_tickets, out, out_lse,
                                  stream);
}
