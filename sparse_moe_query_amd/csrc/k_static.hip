// gqe_forward_static: the forward pass on a workspace the library holds in device memory of its
// own, for callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The workspace is a file-scope device array (`scratch`, GQE_STATIC_SCRATCH_BYTES), one copy per
// GPU the library runs on, held until the process ends.  In host code the array's name is only a
// host-side stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is handed to the kernels.
// Every call on one GPU shares that GPU's array: it keeps the last call's contents (the routing
// statistics gqe_aux_stats reads, the intermediates the backward and the KV export read), and
// calls that overlap on one GPU -- on different streams, or from different handles -- race.
// The forward writes every byte it reads, so nothing needs clearing between calls.
#include <mutex>

#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[GQE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_addr[kMaxDevices] = {};

// The scratch array's device address on the current device (looked up on the first call there).
void* scratch_for(size_t need, size_t* have, int* code) {
    *code = GQE_ERR_WORKSPACE;
    if (need > (size_t)GQE_STATIC_SCRATCH_BYTES) {
        char msg[256];
        snprintf(msg, sizeof(msg),
                 "gqe_forward_static: the shape needs %zu bytes of workspace, the static scratch holds %zu "
                 "(use gqe_forward with a caller workspace)",
                 need, (size_t)GQE_STATIC_SCRATCH_BYTES);
        gqe_set_error(GQE_ERR_WORKSPACE, msg);
        return nullptr;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    *code = GQE_ERR_HIP;
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        gqe_set_error(GQE_ERR_HIP, "gqe_forward_static: no usable current HIP device");
        return nullptr;
    }
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            char msg[256];
            snprintf(msg, sizeof(msg), "gqe_forward_static: hipGetSymbolAddress of the scratch array failed: %s",
                     hipGetErrorString(e));
            gqe_set_error(GQE_ERR_HIP, msg);
            return nullptr;
        }
        g_addr[dev] = p;
    }
    *have = (size_t)GQE_STATIC_SCRATCH_BYTES;
    return g_addr[dev];
}

}  // namespace

extern "C" int gqe_forward_static(gqe_handle_t* h, const void* x, void* y, int64_t batch, int64_t seq, void* stream,
                                  int32_t* route_idx, float* route_w) {
    return gqe_forward_impl(h, x, y, batch, seq, nullptr, 0, stream, route_idx, route_w, scratch_for);
}
