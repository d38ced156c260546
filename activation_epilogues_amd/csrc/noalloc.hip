// convt3d_fused_noalloc: the fused forward pass with the library's own static
// device scratch in place of a caller-provided workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The scratch is a file-scope device array of CONVT3D_NOALLOC_SCRATCH_BYTES.
// Each device the library runs on holds its own copy (the HIP runtime places
// it when the code object is loaded on that device) until the process ends.
// Host code never uses the array's name as an address: at a device's first
// call, with that device current, hipGetSymbolAddress gives that device's
// address of the array, which is kept per device and passed to the kernels as
// the workspace, exactly as convt3d_fused passes the caller's.
#include <hip/hip_runtime.h>

#include <mutex>

#include "convt3d_internal.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[CONVT3D_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` on each device, once looked up

// Address of the current device's scratch (looked up once per device).
int current_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CONVT3D_ERR_LAUNCH;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return CONVT3D_ERR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CONVT3D_OK;
}

}  // namespace

extern "C" int convt3d_fused_noalloc(const float *x, const void *w_packed, const float *bias,
                                     const convt3d_geom *geom, const convt3d_epilogue *epi, float *out,
                                     void *stream) {
    if (!geom || !epi) return CONVT3D_ERR_NULL;
    // workspace of the plan convt3d_fused runs for (geom, epi) right now
    size_t need = 0;
    int st = convt3d::current_plan_workspace(geom, epi, &need);
    if (st) return st;
    if (need > (size_t)CONVT3D_NOALLOC_SCRATCH_BYTES) return CONVT3D_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0 && geom->n > 0) {
        st = current_scratch(&ws);
        if (st) return st;
    }
    // every partial sum and scale / shift in the workspace is written by this
    // call before it is read, so the previous call's contents need no clearing
    return convt3d_fused(x, w_packed, bias, geom, epi, out, ws, need, stream);
}
