// la_prefill_noalloc: la_prefill with its workspace taken from a fixed device array
// instead of a caller buffer, for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this code object (one copy per GPU the library runs on, held
// until the process ends). Host code never passes its name to a kernel: the name is
// a host-side stand-in, not a device address. Its device address is looked up once
// per device with hipGetSymbolAddress, with that device current, on the first call
// made on that device, and only that address is handed on.
#include <mutex>

#include "la_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(LA_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, or null on failure.
void* scratch_address(int dev) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" {

int la_prefill_noalloc(const la_desc* d, const void* q, const void* k, const void* v,
                       const void* g, const void* beta, const float* S0, const float* z0, void* o,
                       float* S_final, float* z_final, void* stream) {
    size_t need = 0;
    const int rc = la_prefill_workspace_size(d, &need);
    if (rc != LA_OK) return rc;
    if (need > kScratchBytes) return LA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
            (void)hipGetLastError();
            return LA_ERR_HIP;
        }
        // the array's address is per device: the stream must run on the current one
        if (stream != nullptr) {
            int sdev = -1;
            if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) {
                (void)hipGetLastError();
                return LA_ERR_HIP;
            }
            if (sdev != dev) return LA_ERR_INVALID;
        }
        ws = scratch_address(dev);
        if (ws == nullptr) return LA_ERR_HIP;
    }
    // The kernels read nothing from the workspace that the same call did not write
    // first, so the array needs no clearing between calls.
    return la_prefill(d, q, k, v, g, beta, S0, z0, o, S_final, z_final, ws, need, stream);
}

}  // extern "C"
