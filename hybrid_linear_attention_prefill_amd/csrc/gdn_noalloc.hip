// gdn_noalloc.hip -- gdn_prefill_chunked_noalloc: the prefill with its workspace in a static
// device array, for callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The array `scratch` below is file-scope device memory: every GPU the library runs on holds
// its own copy (GDN_NOALLOC_WORKSPACE_BYTES) from module load until the process ends.  Host code
// never passes the array's name to a kernel (on the host that name is a stand-in, not a device
// address): on each device's first call, with that device current, hipGetSymbolAddress gives the
// device address, which is kept per device and handed to the prefill as its workspace.  The
// kernels write every workspace byte they read (each sub-chunk's factors are written by the
// first kernel before the second reads them), so nothing needs clearing between calls.  All
// calls on one GPU share the array: calls that overlap in time on one GPU (other streams, other
// threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn_internal.h"

namespace gdn {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of this device's copy of `scratch` (looked up once per device), or null.
void *scratch_address(int dev)
{
    std::call_once(g_once[dev], [dev]() {
        void *p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
    });
    return g_ptr[dev];
}

}  // namespace
}  // namespace gdn

extern "C" gdn_status gdn_prefill_chunked_noalloc(const gdn_desc *desc, const void *x,
                                                  const void *conv_w, const float *g,
                                                  const float *beta, const gdn_state *in,
                                                  gdn_state *out, void *o, int64_t T, int32_t mode,
                                                  int64_t *rows_done, void *stream)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= gdn::kMaxDevices) return GDN_EDEVICE;
    void *ws = gdn::scratch_address(dev);
    if (!ws) return GDN_EDEVICE;
    // every argument check, the size limit (GDN_EWORKSPACE past it) and the launches are those
    // of gdn_prefill_chunked, with the static array as the workspace
    return gdn_prefill_chunked(desc, x, conv_w, g, beta, in, out, o, T, mode, rows_done, ws,
                               (size_t)GDN_NOALLOC_WORKSPACE_BYTES, stream);
}
