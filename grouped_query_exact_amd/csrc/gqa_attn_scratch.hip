// Fixed device-resident workspace of gqa_attn_fwd_noalloc.
//
// Split-KV calls need fp32 partial outputs and log-sum-exps between the
// attention kernel and the combine kernel. gqa_attn_fwd allocates them
// stream-ordered on every call; gqa_attn_fwd_noalloc, for callers that may
// not allocate (graph capture, serving loops that forbid hipMalloc), takes
// them from this file-scope array instead. Every GPU the library runs on
// holds its own copy of kScratchBytes for the life of the process.
//
// In host code `scratch` names a host-side shadow, not device memory: the
// device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress (that device current) and cached; kernels receive that
// address as their workspace argument, exactly as they receive the
// allocated buffer of gqa_attn_fwd.
#include <hip/hip_runtime.h>

#include <mutex>

#include "host_logic.h"
#include "kernels.h"

namespace gqa {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
void* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];
std::once_flag g_scratch_once[kMaxScratchDevices];
}  // namespace

hipError_t scratch_address(int dev, void** ptr) {
    *ptr = nullptr;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    // `dev` is the calling thread's current device (the caller read it with
    // hipGetDevice), so the lookup resolves that device's copy
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_err[dev] = e;
        g_scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
        if (e != hipSuccess) (void)hipGetLastError();
    });
    *ptr = g_scratch_ptr[dev];
    return g_scratch_ptr[dev] ? hipSuccess : (g_scratch_err[dev] != hipSuccess ? g_scratch_err[dev] : hipErrorUnknown);
}

}  // namespace gqa
