// lla_noalloc.hip -- the static device scratch array behind
// lla_prefill_noalloc, for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// The prefill's workspace (one fp32 state per segment per key/value head,
// written by the segment pass and the scan and read by the walks of the same
// call) lives in `scratch`, a file-scope device array of kNoAllocScratchBytes.
// Each device the library runs on holds its own copy until the process ends.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): the first call on a device looks up that
// device's address with hipGetSymbolAddress, with the device current, and
// every later call on the device reuses it.
#include <mutex>

#include "lla_internal.h"

namespace lla {

static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device (null: not looked up)
}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, float** out) {
    int dev = 0;
    hipError_t e;
    if (stream != nullptr) {
        hipDevice_t d = 0;
        if ((e = hipStreamGetDevice(stream, &d)) != hipSuccess) return e;
        dev = (int)d;
    } else if ((e = hipGetDevice(&dev)) != hipSuccess) {
        return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<float*>(g_scratch_ptr[dev]);
    return hipSuccess;
}

}  // namespace lla
