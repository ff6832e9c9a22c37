// gdr_static.hip -- gdr_bwd_static: the backward pass with its workspace in a
// fixed device array of this library instead of a caller buffer, for callers
// that cannot allocate device memory (declared in include/gdr.h).
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdr.h"

namespace gdr {
void set_hip_error(const char* what, hipError_t e);   // gdr_api.cpp
}

namespace {

// The workspace of gdr_bwd_static. Each GPU the code object is loaded on holds
// its own copy until the process ends. In host code this name is a host-side
// stand-in, not a device address: kernels and copies only ever get the address
// hipGetSymbolAddress returns for the current device (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[GDR_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];   // per device: the device address of its `scratch`

// The current device's copy of `scratch`, looked up once per device (with that
// device current) and kept.
int scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        gdr::set_hip_error("hipGetDevice", e);
        return GDR_EHIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return GDR_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            gdr::set_hip_error("hipGetSymbolAddress(scratch)", e);
            return GDR_EHIP;
        }
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return GDR_OK;
}

}  // namespace

extern "C" int gdr_bwd_static(const gdr_bwd_desc_t* d, const void* q, const void* k, const void* v,
                              const float* g, const void* beta, const float* h0, const void* do_,
                              const float* dht, const int32_t* cu_seqlens, void* dq, void* dk, void* dv,
                              float* dg, void* db, float* dh0, void* stream) {
    int rc = gdr_bwd_check(d);
    if (rc != GDR_OK) return rc;
    if (gdr_bwd_workspace_bytes(d) > GDR_STATIC_SCRATCH_BYTES) return GDR_ESCRATCH;
    void* ws = nullptr;
    rc = scratch_ptr(&ws);
    if (rc != GDR_OK) return rc;
    // the workspace needs no clearing: every region is written before it is read
    return gdr_bwd(d, q, k, v, g, beta, h0, do_, dht, cu_seqlens, dq, dk, dv, dg, db, dh0, ws,
                   GDR_STATIC_SCRATCH_BYTES, stream);
}
