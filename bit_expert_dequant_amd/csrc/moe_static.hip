// moe_static.hip -- moe_layer_decode_static: the single-token layer decode with its workspace in a
// file-scope device array instead of caller memory, for callers that cannot allocate (code under
// graph capture, serving loops that forbid allocation).
//
// `scratch` is one array per device (each GPU the library runs on holds its own copy for the life
// of the process).  Its address is taken once per device with hipGetSymbolAddress, with that device
// current, and only that address is handed to kernels: in host code the array's name is a host-side
// stand-in, not a device address.  The array starts zeroed (static storage), which is the state the
// decode workspace needs before its first call; afterwards every call on the device shares it and
// keeps the launch counter and hand-over words of the last call.  Calls on one device that may
// overlap (different streams without ordering) race on it and must not be issued.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "moe_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

std::mutex g_mu;
std::vector<void *> g_ptr;     // device address of `scratch`, per device (nullptr: not taken yet)

int scratch_ptr(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return moe::set_error(MOE_ERR_DEVICE, "hipGetDevice failed");
    std::lock_guard<std::mutex> lock(g_mu);
    if ((int)g_ptr.size() <= dev) g_ptr.resize(dev + 1, nullptr);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return moe::set_error(MOE_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed");
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" int moe_layer_decode_static(const moe_dims *dims, const moe_layer *layers, int n_layers, const void *x,
                                       int x_dtype, unsigned flags, float *out, int32_t *idx, float *w,
                                       void *stream) {
    const size_t need = moe::layer_decode_ws_bytes(dims);
    if (need == 0) return moe::set_error(MOE_ERR_SHAPE, "invalid dims");
    if (need > (size_t)MOE_STATIC_SCRATCH_BYTES)
        return moe::set_error(MOE_ERR_WORKSPACE, "these dims need a decode workspace larger than the static "
                                                 "scratch (MOE_STATIC_SCRATCH_BYTES); use moe_layer_decode");
    void *ws = nullptr;
    if (int s = scratch_ptr(&ws)) return s;
    return moe::layer_decode_entry(dims, layers, n_layers, x, x_dtype, flags, out, idx, w, ws,
                                   (size_t)MOE_STATIC_SCRATCH_BYTES, stream, nullptr, true);
}
