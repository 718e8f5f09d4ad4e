// moe_forward without a caller-provided workspace, for callers that cannot
// allocate device memory: code under HIP graph capture, serving loops that
// must not call hipMalloc, harnesses that forbid it.
//
// The scratch the layer's kernels need (logits, routing weights, histograms,
// the permutation, tile lists, work items, the h and staging rows) comes from
// `scratch`, a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES that every
// GPU the library runs on holds from the moment the library's code is loaded
// on it until the process ends.  In host code the array's name stands for a
// host-side handle, not a device address: its address on the current device
// is looked up once per device with hipGetSymbolAddress and only that
// pointer is passed on.  The kernels need no part of it cleared (every word
// they read in a call is written earlier in the same call), so it is not
// cleared between calls; calls that overlap on one GPU (on different streams
// or threads) share it and race.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

constexpr size_t SCRATCH_BYTES = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;

__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex g_mu;
void *g_scratch[MAX_DEVICES];  // address of `scratch` on each device, once looked up

// The array's address on the current device (looked up on the first call
// there), or null with the error recorded.
void *scratch_on_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        moe::api_fail(MOE_EHIP, "moe_forward_noalloc: no current HIP device");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            char msg[160];
            std::snprintf(msg, sizeof msg, "moe_forward_noalloc: hipGetSymbolAddress: %s",
                          hipGetErrorString(e));
            moe::api_fail(MOE_EHIP, msg);
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int moe_forward_noalloc(const moe_shape_t *shape, const moe_weights_t *w,
                                   const void *x, void *y, int32_t *topk_idx, float *topk_w,
                                   void *stream)
{
    const size_t need = moe_workspace_bytes(shape);
    if (need == 0)  // invalid shape: moe_forward reports which argument
        return moe_forward(shape, w, x, y, topk_idx, topk_w, nullptr, 0, stream);
    if (need > SCRATCH_BYTES) {
        char msg[200];
        std::snprintf(msg, sizeof msg,
                      "moe_forward_noalloc: a pass of this shape needs %zu bytes of scratch, "
                      "the static scratch holds %zu: lower chunk_T",
                      need, SCRATCH_BYTES);
        return moe::api_fail(MOE_EWORKSPACE, msg);
    }
    void *ws = scratch_on_current_device();
    if (!ws)
        return MOE_EHIP;
    return moe_forward(shape, w, x, y, topk_idx, topk_w, ws, SCRATCH_BYTES, stream);
}
