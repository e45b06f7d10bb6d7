// fab_noalloc.hip -- fab_backward_noalloc: fab_backward for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its workspace is a fixed array in the
// library's device memory instead of a caller's buffer; everything else --
// validation, kernels, results -- is fab_backward's.
//
// The array is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy (allocated when the code object is loaded on that device and
// kept until the process ends).  Host code never uses the array's name as an
// address (on the host it only names the variable); its device address on the
// current GPU comes from hipGetSymbolAddress, asked once per device and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fab.h"
#include "fab_launch.h"

static __device__ __align__(256) unsigned char scratch[FAB_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};   // device address of `scratch` on each device, once asked

// Device address of this device's scratch array (hipGetSymbolAddress on first use
// with that device current).
int scratch_ptr(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fab::set_error(FAB_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fab::set_error(FAB_E_UNSUPPORTED, "device index %d beyond the scratch table", dev);
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fab::set_error(FAB_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return FAB_OK;
}

}  // namespace

extern "C" {

int fab_backward_noalloc(const fab_shape *shape, const void *q, const void *k, const void *v,
                         const uint16_t *mask, const void *d, float scale, int mode, const void *O,
                         const float *lse, void *blob, void *stream)
{
    // shape and mode first (host only): the workspace this call needs
    size_t need = 0;
    const int rc = fab_workspace_bytes(shape, mode, mask != nullptr, O != nullptr, &need);
    if (rc != FAB_OK) return rc;
    if (need > (size_t)FAB_NOALLOC_SCRATCH_BYTES)
        return fab::set_error(FAB_E_UNSUPPORTED,
                              "fab_backward_noalloc: this shape needs %zu workspace bytes, above the fixed %zu-byte "
                              "scratch array (fab_backward with a workspace of that size handles it)",
                              need, (size_t)FAB_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    const int rs = scratch_ptr(&ws);
    if (rs != FAB_OK) return rs;
    return fab_backward(shape, q, k, v, mask, d, scale, mode, O, lse, blob, ws, FAB_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
