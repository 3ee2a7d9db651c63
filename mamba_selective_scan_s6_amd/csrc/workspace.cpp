// workspace.cpp - the scan's device workspace: one per (device, stream), cached for the life of
// the process (or until ssm_release_workspaces), grown on demand.
//
// The scan's workgroups exchange segment aggregates and inclusive states through it. Flags in it
// carry the launch's epoch, so it never needs clearing between launches: a new launch on the same
// workspace takes the next epoch and ignores every flag written under an older one. It is zeroed
// when allocated and again when the 30-bit epoch wraps. Word 0 collects error flags that kernels
// raise (a bounded cross-workgroup wait that timed out).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <functional>
#include <map>
#include <mutex>
#include <utility>

#include "ssm_kernels.hpp"

namespace ssm {
namespace {

struct Entry {
    void* ptr = nullptr;
    size_t bytes = 0;
    uint32_t epoch = 0;
};

std::mutex g_mu;
std::map<std::pair<int, uintptr_t>, Entry> g_ws;

constexpr uint32_t kEpochMax = (1u << 30) - 1;

}  // namespace

hipError_t with_scan_workspace(hipStream_t stream, size_t bytes,
                               const std::function<hipError_t(void*, uint32_t)>& launch) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_mu);
    Entry& w = g_ws[{dev, reinterpret_cast<uintptr_t>(stream)}];
    if (w.bytes < bytes) {
        if (w.ptr) {
            // the old buffer may still be in use by work queued on this stream
            if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
            if ((e = hipFree(w.ptr)) != hipSuccess) return e;
            w.ptr = nullptr;
            w.bytes = 0;
        }
        const size_t grow = bytes + bytes / 4;
        const size_t want = (grow + (size_t(1) << 20) - 1) & ~((size_t(1) << 20) - 1);
        if ((e = hipMalloc(&w.ptr, want)) != hipSuccess) {
            w.ptr = nullptr;
            return e;
        }
        w.bytes = want;
        w.epoch = 0;
        if ((e = hipMemsetAsync(w.ptr, 0, want, stream)) != hipSuccess) return e;
    }
    if (w.epoch >= kEpochMax) {
        if ((e = hipMemsetAsync(w.ptr, 0, w.bytes, stream)) != hipSuccess) return e;
        w.epoch = 0;
    }
    // the launch is enqueued under the lock, so no other caller can free or regrow this buffer
    // between choosing it and using it
    return launch(w.ptr, ++w.epoch);
}

hipError_t take_workspace_errors(hipStream_t stream, uint32_t* flags) {
    *flags = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_ws.find({dev, reinterpret_cast<uintptr_t>(stream)});
    if (it == g_ws.end() || !it->second.ptr) return hipSuccess;
    uint32_t v = 0;
    if ((e = hipMemcpy(&v, it->second.ptr, sizeof(v), hipMemcpyDeviceToHost)) != hipSuccess) return e;
    if (v) {
        const uint32_t zero = 0;
        if ((e = hipMemcpy(it->second.ptr, &zero, sizeof(zero), hipMemcpyHostToDevice)) != hipSuccess) return e;
    }
    *flags = v;
    return hipSuccess;
}

hipError_t release_workspaces() {
    std::lock_guard<std::mutex> lock(g_mu);
    hipError_t first = hipSuccess;
    if (!g_ws.empty()) first = hipDeviceSynchronize();
    for (auto& kv : g_ws) {
        if (kv.second.ptr) {
            int cur = 0;
            hipError_t e = hipGetDevice(&cur);
            if (e == hipSuccess) e = hipSetDevice(kv.first.first);
            if (e == hipSuccess) e = hipFree(kv.second.ptr);
            const hipError_t r = hipSetDevice(cur);
            if (first == hipSuccess) first = e != hipSuccess ? e : r;
        }
    }
    g_ws.clear();
    return first;
}

}  // namespace ssm
