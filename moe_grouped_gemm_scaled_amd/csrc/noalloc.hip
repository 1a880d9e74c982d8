// noalloc.hip -- the split-K scratch of dg_fp8_gemm_nt_noalloc, for callers
// that cannot allocate device memory (code under graph capture, serving loops
// that forbid allocation).
//
// The scratch is one file-scope device array per GPU, loaded with the code
// object and held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the
// first call on each device looks up the array's device address with
// hipGetSymbolAddress, with that device current, and every call then passes
// that address.  The layout is the one every split-K launcher uses (int32
// arrival counters first, then fp32 partials).  The counters start at zero
// (static storage is zero-filled when the code object is loaded; the first
// call also clears them with a fill kernel when its stream is not being
// captured) and every call that completes leaves them zero, so calls in
// stream order can share the array.  Calls that overlap on one GPU race.
#include <mutex>

#include "dg_internal.h"

namespace dg {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Clears `n` 32-bit words at p (a kernel rather than a memset node, so that
// the clear is safe inside captured graphs as well).
__global__ void __launch_bounds__(256) clear_words(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void **ptr, size_t *bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [&] {
        void *p = nullptr;
        hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (r == hipSuccess && p == nullptr) r = hipErrorInvalidSymbol;
        if (r == hipSuccess) {
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            r = hipStreamIsCapturing(stream, &cs);
            if (r == hipSuccess && cs == hipStreamCaptureStatusNone) {
                const size_t words = kSplitCounterBytes / 4;
                hipLaunchKernelGGL(clear_words, dim3(16), dim3(256), 0, stream, static_cast<uint32_t *>(p), words);
                r = hipGetLastError();
            }
        }
        g_scratch_ptr[dev] = r == hipSuccess ? p : nullptr;
        g_scratch_err[dev] = r;
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    *ptr = g_scratch_ptr[dev];
    *bytes = kNoallocScratchBytes;
    return hipSuccess;
}

}  // namespace dg
