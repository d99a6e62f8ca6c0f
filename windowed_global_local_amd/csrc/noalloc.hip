// noalloc.hip -- atlas_hier_attn_bwd_noalloc: the attention backward with its
// workspace (the per-query D rows) in a fixed device array instead of a
// caller-supplied buffer, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy, at its own address, from the code object's load until
// the process ends.  In host code the array's name is only a host-side
// stand-in, so its device address is looked up once per device (with that
// device current) and only that address is ever handed to kernels.
#include "atlas.h"
#include "atlas_internal.hpp"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr int64_t kScratchBytes = ATLAS_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (null: not looked up)

// Device address of the current device's copy of `scratch`.
int current_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        atlas::note_hip_error((int)e);
        return ATLAS_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        atlas::note_hip_error((int)hipErrorInvalidDevice);
        return ATLAS_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            atlas::note_hip_error((int)(e != hipSuccess ? e : hipErrorInvalidSymbol));
            return ATLAS_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ATLAS_OK;
}

}  // namespace

extern "C" int atlas_hier_attn_bwd_noalloc(
    void *dq_d, void *dk_d, void *dv_d, void *dq_g, void *dk_g, void *dv_g, const void *q_d,
    const void *k_d, const void *v_d, const void *q_g, const void *k_g, const void *v_g,
    const void *o_d, const void *o_g, const void *do_d, const void *do_g, const float *lse_detail,
    const float *lse_global, atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, int32_t heads,
    int32_t head_dim, float softmax_scale, int32_t dtype, void *stream)
{
    return atlas::hier_attn_bwd_scratch(dq_d, dk_d, dv_d, dq_g, dk_g, dv_g, q_d, k_d, v_d, q_g, k_g,
                                        v_g, o_d, o_g, do_d, do_g, lse_detail, lse_global,
                                        current_scratch, kScratchBytes, grid, cube, gproxy, heads,
                                        head_dim, softmax_scale, dtype, stream);
}
