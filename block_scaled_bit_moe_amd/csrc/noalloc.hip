// noalloc.hip -- the workspace of moe_layer_decode_noalloc: a file-scope
// device array instead of caller memory, for callers that cannot allocate.
//
// Each GPU holds its own copy of `scratch` (allocated when the library's code
// object is loaded on that GPU, kept until the process ends).  In host code
// the array's name is only a host-side stand-in, so its device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and only that address is ever handed to a kernel.
#include <mutex>

#include "kernels.h"

namespace moeq {

static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_mu;
void *g_ptr[NOALLOC_MAX_DEVICES];     // device address of `scratch`, per device
bool g_ready[NOALLOC_MAX_DEVICES];    // cleared once
}  // namespace

__global__ void noalloc_clear_kernel(uint4 *p, size_t n16) {
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = z;
}

// The current device's scratch address in *ptr.  On the first call on a
// device the address is looked up and the whole array is cleared with a fill
// kernel on `s` (ahead of the caller's kernels on the same stream); that
// first call may not be made while `s` is being captured into a graph.
hipError_t noalloc_workspace(hipStream_t s, void **ptr, const char **why) {
    *ptr = nullptr;
    *why = "";
    const int dev = current_device();
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) {
        *why = "device ordinal beyond the library's table";
        return hipErrorInvalidDevice;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ready[dev]) {
        hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(s, &st);
        if (e != hipSuccess) return e;
        if (st != hipStreamCaptureStatusNone) {
            *why = "the first call on a device clears the static workspace and may not be captured";
            return hipErrorStreamCaptureUnsupported;
        }
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(noalloc_clear_kernel, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint4 *>(p),
                           (size_t)NOALLOC_SCRATCH_BYTES / 16);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
        g_ready[dev] = true;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace moeq
