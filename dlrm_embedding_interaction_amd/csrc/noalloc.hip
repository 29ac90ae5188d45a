// noalloc.hip -- dlrm_forward without a caller-provided workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The workspace of dlrm_forward (R = [x | Z] and two hidden buffers; see
// make_plan in api.hip) lives instead in one file-scope device array of
// kNoAllocScratchBytes.  Each GPU the library runs on holds its own copy of
// the array until the process ends.  Host code never uses the array's name as
// an address (in host code it is only a stand-in): the first call on a device
// asks the runtime for that device's address with hipGetSymbolAddress, once,
// with the device current, and every later call on that device passes the
// address kept for it.  Nothing here allocates or frees memory.
//
// Every call on one GPU shares that GPU's array: calls that overlap in time
// on one GPU (different streams, or different host threads) race on it.  The
// forward writes every workspace element it later reads, so the array needs
// no clearing between calls.
#include <mutex>

#include "dlrm_internal.h"

#define DLRM_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// This device's address of `scratch` (looked up once per device), or NULL.
hipError_t scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [dev] {
        void* p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
    });
    *out = g_ptr[dev];
    return g_ptr[dev] ? hipSuccess : (g_err[dev] != hipSuccess ? g_err[dev] : hipErrorInvalidValue);
}

}  // namespace

DLRM_API size_t dlrm_forward_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

DLRM_API dlrm_status_t dlrm_forward_noalloc(const dlrm_model_t* m, int64_t batch, const float* dense,
                                            const void* const* indices, const int64_t* n_indices,
                                            const void* const* offsets, int32_t index_bytes, float* out,
                                            void* stream) {
    const size_t need = dlrm_forward_workspace_bytes(m, batch);
    // an invalid model or batch: dlrm_forward reports which check fails, before any launch
    if (need == 0) return dlrm_forward(m, batch, dense, indices, n_indices, offsets, index_bytes, out, nullptr, 0,
                                       stream);
    if (need > kNoAllocScratchBytes) return DLRM_E_UNSUPPORTED;
    void* ws = nullptr;
    if (scratch_for_current_device(&ws) != hipSuccess) return DLRM_E_HIP;
    return dlrm_forward(m, batch, dense, indices, n_indices, offsets, index_bytes, out, ws, kNoAllocScratchBytes,
                        stream);
}
