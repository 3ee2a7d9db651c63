// noalloc.hip - the scan workspace of the entry point that allocates nothing
// (ssm_scan_fwd_noalloc): a file-scope device array, one copy per GPU the library runs on, held
// until the process ends.
//
// In host code the array's name is only a host-side stand-in, not a device address. Its address on
// each device is looked up once with hipGetSymbolAddress (with that device current) and kept, and
// only that address is handed to kernels. On its first use on a device the array is cleared by a fill
// kernel (no hipMemset, so the first call may also be captured in a graph); from then on the scan
// kernels leave it ready for the next call, as they do a caller's workspace.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "ssm_kernels.hpp"

namespace ssm {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevicesNA = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevicesNA] = {};
bool g_cleared[kMaxDevicesNA] = {};

__global__ __launch_bounds__(256) void clear_kernel(uint4* p, int64_t n) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

hipError_t noalloc_workspace(hipStream_t stream, void** ws) {
    *ws = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevicesNA) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    if (!g_cleared[dev]) {
        hipLaunchKernelGGL(clear_kernel, dim3(1024), dim3(256), 0, stream, static_cast<uint4*>(g_ptr[dev]),
                           static_cast<int64_t>(kNoAllocScratchBytes / 16));
        if ((e = hipGetLastError()) != hipSuccess) return e;
        g_cleared[dev] = true;
    }
    *ws = g_ptr[dev];
    return hipSuccess;
}

}  // namespace ssm
