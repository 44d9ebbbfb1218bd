// bi_linear_backward_static: bi_linear_backward for callers that cannot
// allocate device memory.  The f32 dW chunk partials, the only scratch memory
// of the backward, live in a file-scope device array of a fixed size that the
// library owns; each GPU the library runs on holds its own copy until the
// process ends.  Host code reaches that copy only through the device address
// that hipGetSymbolAddress returns for the current device (looked up once per
// device, on the first call there); the array's name itself is never used as
// an address on the host.
#include "../../include/bi.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr size_t kScratchBytes = BI_STATIC_SCRATCH_BYTES;

// f32 partials [chunks][k][n] of the chunked dW; every call overwrites all of
// the partials it reads, so nothing has to start at zero
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// device address of the current GPU's copy of `scratch`
int scratch_address(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BI_ERR_HIP;
    std::call_once(g_once[dev], [dev] {
        g_err[dev] = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch));
    });
    if (g_err[dev] != hipSuccess || g_ptr[dev] == nullptr) return BI_ERR_HIP;
    *ptr = g_ptr[dev];
    return BI_OK;
}

}  // namespace

extern "C" int bi_linear_backward_static(void *dx, void *dw, const void *dy, const void *x,
                                         const void *w, int64_t m, int64_t k, int64_t n,
                                         int dtype, hipStream_t stream, int tc) {
    // the partials this call needs (0 for an invalid argument, which the full
    // validation of bi_linear_backward below then reports)
    const size_t need = dw ? bi_backward_dw_workspace_bytes(m, k, n, dtype, tc) : 0;
    if (need > kScratchBytes) return BI_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        const int st = scratch_address(&ws);
        if (st != BI_OK) return st;
    }
    return bi_linear_backward(dx, dw, dy, x, w, m, k, n, dtype, ws, need, stream, tc);
}
