// lookback.hpp - the cross-workgroup workspace of the scan kernels (gfx950): its layout, the tag
// that marks one launch's publications, and the publication and polling primitives.
//
// The sequence of each channel group (64 channels of one batch row) is cut into segments, one per
// workgroup. A segment publishes its affine aggregate (the state it produces from a zero state, and
// the sum of its steps) and later its inclusive state (the state at its end); a successor folds
// aggregates until it reaches an inclusive state ("Module 19: State-Space Models (Mamba)", The
// Parallel Scan: composing affine steps is associative).
//
// Workspace layout (bytes; the caller owns it and zero-fills it once before its first use):
//   [0, 256)                  header: word 0 sticky error flags, 64-bit word 1 the launch tag,
//                             word 4 the count of channel groups done looking back in this launch
//   256 + k * kSlotBytes      slot k: a 64-bit flag (in a row of its own), then the aggregate (16
//                             states + step sum, each a row of 64 channels), then the inclusive state
//                             (16 rows of 64)
// The slot stride does not depend on the problem, so a flag word is only ever written as a flag,
// whatever shapes earlier launches on the same workspace had.
//
// Launch tag. Every workgroup reads the tag from the header when it starts and writes its flags as
// (tag << 2) | status, so flags left by earlier launches never match. The last segment of each
// channel group counts its group as done once its look-back has finished: by then every segment of
// the group has published something, so it has read the tag. The workgroup that counts the last
// group advances the tag and clears the count; the next launch on the stream reads the new tag.
// Nothing on the host keeps state, and a replayed graph advances the tag like a fresh launch.
//
// Memory ordering. Published values and flags are written and read with agent-scope relaxed atomic
// accesses, which on gfx950 are stores and loads with the sc1 bit: they bypass the per-XCD L2's
// non-coherent state and are performed at the device's coherence point. A publishing wave waits for
// its stores to complete (s_waitcnt vmcnt(0)) before the workgroup barrier that precedes the flag
// store, and a reader issues its data loads only after the flag load has returned. This is the
// release and acquire sequence the compiler emits for agent scope on gfx950 without its L2
// write-back and invalidate, which only serve non-atomic (cached) accesses; the data here is never
// accessed non-atomically.
#pragma once

#include "ssm_device.hpp"

namespace ssm {
namespace lb {

constexpr size_t kHeaderBytes = 256;
constexpr int kRow = 64 * 4;                    // one row of 64 channels, fp32
constexpr int kAggRows = kMaxState + 1;         // H for 16 states, then the step sum
constexpr size_t kSlotBytes = kRow * (1 + kAggRows + kMaxState);  // flag row + aggregate + inclusive
constexpr uint32_t kStatusAgg = 1;
constexpr uint32_t kStatusIncl = 2;
constexpr int kDefaultSpinLimit = 200000;       // polls (each with a short sleep), about 0.1 s

__host__ __device__ constexpr size_t workspace_bytes(int64_t slots) {
    return kHeaderBytes + static_cast<size_t>(slots) * kSlotBytes;
}

struct Header {
    uint32_t error;     // sticky flags: 1 = a bounded wait timed out
    uint32_t pad0;
    uint64_t tag;       // launch tag (flags of this launch carry it)
    uint32_t groups_done;
};

__device__ __forceinline__ Header* header(char* ws) { return reinterpret_cast<Header*>(ws); }
__device__ __forceinline__ char* slot(char* ws, int64_t k) { return ws + kHeaderBytes + k * static_cast<int64_t>(kSlotBytes); }
__device__ __forceinline__ uint64_t* flag(char* ws, int64_t k) { return reinterpret_cast<uint64_t*>(slot(ws, k)); }
__device__ __forceinline__ float* agg(char* ws, int64_t k) { return reinterpret_cast<float*>(slot(ws, k) + kRow); }
__device__ __forceinline__ float* incl(char* ws, int64_t k) {
    return reinterpret_cast<float*>(slot(ws, k) + kRow * (1 + kAggRows));
}

__device__ __forceinline__ float ld(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_flag(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's memory accesses have completed (published stores are then performed).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

// The launch tag, read once per workgroup.
__device__ __forceinline__ uint64_t read_tag(char* ws) {
    return __hip_atomic_load(&header(ws)->tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by one thread of a channel group's last segment once its look-back has finished. The
// thread that counts the last of `ngroups` groups advances the tag for the next launch.
__device__ __forceinline__ void group_done(char* ws, uint64_t tag, uint32_t ngroups) {
    Header* h = header(ws);
    const uint32_t prev = __hip_atomic_fetch_add(&h->groups_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1 == ngroups) {
        __hip_atomic_store(&h->groups_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&h->tag, tag + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ __forceinline__ void raise_error(char* ws, uint32_t bits) {
    __hip_atomic_fetch_or(&header(ws)->error, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Decoupled look-back by one wave: find the nearest predecessor j < s of the channel group with a
// published inclusive state (-1: the zero initial state), polling up to 64 flags per round (lane i
// looks at s - 1 - i). `base` is the group's first slot. If `publish_agg` is given and a predecessor
// has not published yet, it is called once (by every lane) before waiting, so that successors can
// fold past this segment. Returns -1 also on timeout, after raising the error flag.
template <typename PublishAgg>
__device__ __forceinline__ int64_t look_back(char* ws, int64_t base, int64_t s, uint64_t tag, int spin_limit,
                                             bool published, PublishAgg&& publish_agg) {
    const int lane = threadIdx.x & 63;
    int64_t jhi = s - 1;
    int spins = 0;
    for (;;) {
        const int64_t j = jhi - lane;  // lane 0 = nearest predecessor
        uint32_t status = kStatusIncl;  // before the first segment: the zero state counts as inclusive
        if (j >= 0) {
            const uint64_t f = ld_flag(flag(ws, base + j));
            status = (f >> 2) == tag ? static_cast<uint32_t>(f & 3u) : 0u;
        }
        const uint64_t incl_mask = __ballot(status == kStatusIncl);
        const uint64_t none_mask = __ballot(status == 0u);
        const int first = incl_mask ? __builtin_ctzll(incl_mask) : 64;
        const uint64_t before = first >= 64 ? ~0ull : ((1ull << first) - 1ull);
        if (none_mask & before) {  // a predecessor has not published yet: wait
            if (!published) {
                publish_agg();
                published = true;
            }
            if (++spins > spin_limit) {
                if (lane == 0) raise_error(ws, 1u);
                return -1;
            }
            __builtin_amdgcn_s_sleep(2);
            continue;
        }
        if (first < 64) return jhi - first;
        jhi -= 64;  // 64 aggregates in a row: keep looking further back
    }
}

}  // namespace lb
}  // namespace ssm
