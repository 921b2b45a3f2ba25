// api_noalloc.hip -- plora_backward_dAdB_noalloc: the weight-gradient entry
// point for callers that cannot allocate device memory (code under HIP graph
// capture, serving loops, harnesses that forbid hipMalloc).
//
// The workspace of plora_backward_dAdB (fp32 partial sums of adapters whose
// tokens span several chunks, and the bf16 hi/lo transposes of H and G) lives
// in a file-scope device array of kScratchBytes instead of a caller buffer.
// Each device holds its own copy of the array for as long as the process
// runs; its address on a device is taken once, with that device current, by
// hipGetSymbolAddress and kept per device (in host code the array's name is
// not a device address).  The kernels write every scratch byte they read
// before reading it, so no call needs it cleared, and calls on one device
// share it: two calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string>

#include "api_util.h"
#include "plora.h"

namespace {

constexpr size_t kScratchBytes = PLORA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device (looked up once per
// device); nullptr with *err set on failure.
void* scratch_on_current_device(hipError_t* err, int* dev_out) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    *dev_out = dev;
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" int plora_backward_dAdB_noalloc(const plora_desc* d, const void* X, const void* dY, const float* H,
                                           const float* G, float* dA, float* dB, int accumulate, void* stream) {
    try {
        // an invalid descriptor: the workspace entry point reports it (nothing enqueued)
        if (plora_validate(d) != PLORA_OK)
            return plora_backward_dAdB_acc(d, X, dY, H, G, dA, dB, nullptr, 0, accumulate, stream);
        const size_t need = plora_workspace_bytes(d);
        if (need > kScratchBytes)
            return plora::fail(PLORA_ERR_WORKSPACE, "this problem needs " + std::to_string(need) +
                                                        " bytes of scratch; the no-allocation entry point holds " +
                                                        std::to_string(kScratchBytes));
        void* ws = nullptr;
        if (need > 0) {
            hipError_t e = hipSuccess;
            int dev = 0;
            ws = scratch_on_current_device(&e, &dev);
            if (!ws) return plora::hip_fail(e, ("scratch address on device " + std::to_string(dev)).c_str());
        }
        return plora_backward_dAdB_acc(d, X, dY, H, G, dA, dB, ws, need, accumulate, stream);
    } catch (...) {
        return plora::fail(PLORA_ERR_HIP, "unexpected exception");
    }
}
