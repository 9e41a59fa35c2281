// kda_noalloc.hip -- kda_chunk_fwd for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc): the two-kernel schedule's scratch comes from a static device
// array of the library instead of a caller-supplied workspace.
#include "../../include/kda.h"
#include "kda_internal.h"

#include <mutex>

namespace {

// One copy per GPU, alive until the process ends.  In host code `scratch` is
// a host-side stand-in for the symbol, not a device address: only the pointer
// returned by hipGetSymbolAddress (per device) is handed to kernels.
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::once_flag g_once[kMaxDevices];
hipError_t g_status[kMaxDevices];

}  // namespace

// Device address of this device's copy of `scratch` (looked up once per
// device, with that device current), or nullptr with *err set.
void* kda::noalloc_scratch(hipError_t* err)
{
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) { *err = hipErrorInvalidDevice; return nullptr; }
    std::call_once(g_once[dev], [dev]() {
        void* p = nullptr;
        g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch[dev] = g_status[dev] == hipSuccess ? p : nullptr;
    });
    *err = g_status[dev];
    return g_scratch[dev];
}

extern "C" int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                     const float* log_alpha, int gate, const void* beta, const float* S0,
                                     void* o, float* S_T, int B, int T, int H, int dk, int dv, int dtype,
                                     void* stream)
{
    // The scratch of the schedule kda_chunk_fwd_gated runs with its preferred
    // workspace, else of the one-pass scan; a shape that needs more than the
    // array is rejected.  (Invalid shapes ask for nothing and fail validation.)
    size_t need = kda_chunk_fwd_workspace_size(B, T, H, dk, dv, dtype);
    if (need > KDA_NOALLOC_SCRATCH_BYTES) {
        need = kda_chunk_fwd_scan_workspace_size(B, T, H, dk, dv, dtype);
        if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
    }
    // Same validation and kernels as kda_chunk_fwd_gated; the scratch
    // pointer is looked up only after the arguments have passed validation.
    return kda::chunk_fwd_entry(q, k, v, log_alpha, gate, beta, S0, o, S_T, B, T, H, dk, dv, dtype, nullptr,
                                0, need, stream);
}
