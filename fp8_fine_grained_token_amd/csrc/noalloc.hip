// The block-scaled GEMM for callers that cannot allocate device memory: its
// split-K partial sums go to a file-scope device array instead of a caller
// workspace.
//
// Every GPU that loads this library holds its own copy of `scratch` until
// the process ends.  In host code the array's name is only a host-side
// stand-in, never a device address: the device address is looked up once
// per device with hipGetSymbolAddress (with that device current) and cached,
// and only that address is handed to the kernels.  All calls on one GPU
// share its array, so calls that overlap in time on one GPU (different
// streams, or different host threads) race on it.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "launch.hpp"

namespace fp8blk {

namespace {

// Split-K partials of the small-tile plan: at most 256 workgroups of 128 x
// 64 FP32 outputs each, so every plan fits in 8 MiB.
constexpr size_t kScratchBytes = (size_t)8 << 20;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Device address of this device's copy of `scratch`, looked up the first
// time the device is seen (with it current) and cached.
hipError_t scratch_for_stream(hipStream_t stream, void **out) {
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t launch_block_gemm_noalloc(const void *a, const float *sa, const void *w,
                                     const float *sw, void *c, bool bf16_out, int64_t M,
                                     int64_t N, int64_t K, hipStream_t stream) {
    const size_t need = gemm_workspace_bytes(M, N, K);
    void *ws = nullptr;
    if (need > 0) {
        const hipError_t e = scratch_for_stream(stream, &ws);
        if (e != hipSuccess) return e;
    }
    // The partials need no initialization: every split writes its whole
    // tile before the reduction reads it.
    return launch_block_gemm(a, sa, w, sw, c, bf16_out, M, N, K, ws, need, false, stream);
}

}  // namespace fp8blk
