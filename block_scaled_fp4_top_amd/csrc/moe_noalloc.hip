// moe_forward for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the same launch
// sequence on a workspace that lives in a file-scope device array of the
// library instead of a caller buffer.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends. Host code never passes the array's name to a kernel or a copy:
// in host code that name is a host-side stand-in, not a device address. The
// array's address on a device comes from hipGetSymbolAddress, looked up once
// per device with that device current, and only that address is used.
#include <mutex>

#include "moe_internal.h"
#include "moe_kernels.h"

namespace moe {
constexpr size_t kNoallocScratchBytes = 64ull << 20;  // 64 MiB
}

static __device__ __align__(256) uint8_t scratch[moe::kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device

// The address of this device's copy of `scratch` (the current device's),
// looked up on the first call on that device.
int scratch_on_current_device(void** out) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return moe::report_error(MOE_ERR_HIP, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return moe::report_error(MOE_ERR_UNSUPPORTED, "device index above 63");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (r != hipSuccess || !p)
            return moe::report_error(MOE_ERR_HIP, r != hipSuccess ? hipGetErrorString(r)
                                                                  : "no device address for the scratch array");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}
}  // namespace

extern "C" int moe_forward_noalloc(const moe_dims* d, const void* prepared, size_t prepared_bytes,
                                   const uint16_t* x, const float* logits, int32_t T, int32_t K,
                                   int32_t mode, int32_t act, int32_t router_weight_on_input,
                                   int32_t deterministic_finalize, uint16_t* y,
                                   hipStream_t stream) {
    int rc = moe::forward_checked(d, prepared, prepared_bytes, x, logits, T, K, mode, act,
                                  router_weight_on_input, deterministic_finalize, y);
    if (rc) return rc;
    const size_t need = moe::forward_workspace_bytes(d, T, K, mode);
    if (need > moe::kNoallocScratchBytes) {
        char msg[160];
        snprintf(msg, sizeof msg, "this forward needs %zu bytes of workspace; the built-in one holds %zu",
                 need, (size_t)moe::kNoallocScratchBytes);
        return moe::report_error(MOE_ERR_WORKSPACE, msg);
    }
    void* ws = nullptr;
    rc = scratch_on_current_device(&ws);
    if (rc) return rc;
    return moe::enqueue_forward(d, prepared, x, logits, T, K, mode, act, router_weight_on_input,
                                deterministic_finalize, ws, y, stream);
}
