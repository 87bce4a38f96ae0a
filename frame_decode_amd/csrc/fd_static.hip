// fd_step_static: the decode step with the library's own device scratch as
// its workspace, for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array; in host code its name is only a
// stand-in for the symbol, so its device address is resolved once per GPU
// with hipGetSymbolAddress (with that GPU current) and only that address is
// handed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fd.h"
#include "fd_internal.h"

static __device__ __align__(256) uint8_t scratch[FD_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this GPU's copy of `scratch` (resolved on first use).
hipError_t scratch_on(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" fd_status fd_step_static(fd_ctx* ctx, const void* x_in, void* y_out, void* depth_out,
                                    void* stream) {
    if (!ctx) return FD_E_INVAL;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != fd::ctx_device(ctx)) return FD_E_INVAL;
    void* ws = nullptr;
    if (scratch_on(dev, &ws) != hipSuccess) return FD_E_DEVICE;
    return fd::step_on_workspace(ctx, ws, FD_STATIC_SCRATCH_BYTES, x_in, y_out, depth_out, stream);
}
