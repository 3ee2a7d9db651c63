// ssm_kernels.hpp - launch interface between the C ABI shim and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// ceil(a / b) for a >= 0 and b > 0, without the overflow of (a + b - 1) / b near INT64_MAX.
__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0 ? 1 : 0); }
// a * b for a, b >= 0, saturating at INT64_MAX (size checks compare the result with a limit).
__host__ __device__ constexpr int64_t sat_mul(int64_t a, int64_t b) {
    return a != 0 && b > INT64_MAX / a ? INT64_MAX : a * b;
}

struct ScanArgs {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;           // nullable
    const void* z;            // nullable
    const float* delta_bias;  // nullable
    void* out;
    float* last_state;        // nullable
    int64_t nb, nd, L;
    int N;
    int softplus;
    int zoh;  // exact zero-order-hold input gain (else Euler, Delta B)
    float* hblk = nullptr;  // checkpoint pass: state entering each 16-token block, [nb, nd, ceil(L/16), 16]
    int out_f32 = 0;        // out is fp32 whatever the input type
    // checkpoint pass, the adjoint's block pass of the backward: dout (io dtype, [nb, nd, L]) in; per
    // 16-token block the reverse aggregate of the blocks after it in its 64-token segment (the adjoint
    // carried from zero at the segment's end to the block's end), [nb * groups, segments, 4, 16, 64], and
    // their sum of steps, [nb * groups, segments, 4, 64], out
    const void* dout = nullptr;
    float* lam = nullptr;
    float* sdt = nullptr;
    float* segagg = nullptr;  // per 64-token segment of each 64-channel group: its blocks' aggregates composed,
                              // [nb * groups, segments, 17, 64] (16 states, then the step sum)
};

struct UpdateArgs {
    float* state;
    const void* x;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;  // nullable
    const void* z;   // nullable
    void* out;
    int64_t nb, nd;
    int N;
    int zoh;  // exact zero-order-hold input gain (else Euler, Delta B)
    int out_f32 = 0;  // out is fp32 whatever the input type
};

// Backward of the scan: the forward inputs, dout, the gradient outputs and the scratch buffers
// (carved from the stream workspace by launch_scan_bwd).
struct BwdArgs {
    ScanArgs a;              // forward inputs; a.out, a.last_state unused
    const void* dout;        // [nb, nd, L] io dtype
    void* du;                // [nb, nd, L] io dtype
    void* ddelta;            // [nb, nd, L] io dtype
    void* dz;                // [nb, nd, L] io dtype, used iff a.z
    float* dA;               // [nd, N]
    float* dB;               // [nb, L, N]
    float* dC;               // [nb, L, N]
    float* dD;               // [nd], nullable
    float* dbias;            // [nd], nullable
    // scratch
    float* hblk = nullptr;   // [nb, nd, nblk, 16] state entering each 16-token block
    float* lam = nullptr;    // [nb * groups, nseg, 4, 16, 64] reverse aggregate of the blocks after each
                             // block in its segment, from a zero carry at the segment's end
    float* sdt = nullptr;    // [nb * groups, nseg, 4, 64] those blocks' sum of steps
    float* segagg = nullptr;    // [nb * groups, nseg, 17, 64] segment reverse aggregates (16 states, step sum)
    float* segcarry = nullptr;  // [nb * groups, nseg, 16, 64] adjoint carry into each segment from the right
    float* dBp = nullptr;    // [groups, nb, L, 16] dB partials per 64-channel group
    float* dCp = nullptr;    // [groups, nb, L, 16]
    float* dAp = nullptr;    // [nb, nseg, nd, 16] dA partials per 64-token segment
    float* dDp = nullptr;    // [nb, nseg, nd]
    float* dbp = nullptr;    // [nb, nseg, nd]
    int64_t groups = 0, nbg = 0, nblk = 0, nseg = 0;
};

// Extra workspace bytes of a backward call (beyond scan_workspace_bytes), and the launch: the
// two-sweep forward in checkpoint mode on `scan_workspace`, then the backward kernels on `extra`.
size_t scan_bwd_extra_bytes(int64_t nb, int64_t nd, int64_t L);
hipError_t launch_scan_bwd(BwdArgs q, bool io_bf16, void* scan_workspace, void* extra, hipStream_t stream);

constexpr int kMaxConvWidth = 8;  // largest causal convolution width the kernels take

struct ConvArgs {
    const void* x;          // [nb, nd, L] (sequence) or [nb, nd] (window step), io dtype
    const float* w;         // [nd, K]
    const float* bias;      // [nd], nullable
    void* out;              // like x
    float* window;          // [nb, nd, K], window step only
    int64_t nb, nd, L;      // L unused by the window step
    int K;
    int silu;
};

// Causal depthwise convolution + SiLU over a sequence, and its one-token window update.
int64_t conv_max_blocks(int64_t nb, int64_t nd, int64_t L);
hipError_t launch_causal_conv1d(const ConvArgs& a, bool io_bf16, hipStream_t stream);
hipError_t launch_conv_window_update(const ConvArgs& a, bool io_bf16, hipStream_t stream);

// Workspace bytes of a scan (lookback.hpp: a header and one slot per segment of each channel group),
// and the number of workgroups one launch uses.
size_t scan_workspace_bytes(int64_t nb, int64_t nd, int64_t L);
int64_t scan_max_blocks(int64_t nb, int64_t nd, int64_t L);
// Tokens per workgroup segment of the scan kernels.
int scan_segment_tokens(int64_t nb, int64_t nd, int64_t L);

// io_bf16: false = fp32 io tensors, true = bf16 io tensors. Arguments are validated by the caller.
// workspace: at least scan_workspace_bytes() device bytes, zero-filled before its first use and not
// used by another launch that may run at the same time.
hipError_t launch_scan_fwd(const ScanArgs& a, bool io_bf16, void* workspace, hipStream_t stream);
// The backward's checkpoint pass (scan_ckpt.hip): the state entering every 16-token block into a.hblk.
hipError_t launch_scan_ckpt(const ScanArgs& a, bool io_bf16, void* workspace, hipStream_t stream);
// Polls a scan's look-back may wait before recording a timeout (<= 0: the default); returns the previous.
int set_scan_wait_limit(int polls);
int scan_wait_limit();
hipError_t launch_state_update(const UpdateArgs& a, bool io_bf16, hipStream_t stream);

// Mamba-2 scan with a scalar decay per head (ssd.hip). x, y: [nb, L, heads, P]; a: [nb, L, heads]
// fp32; b, c: [nb, L, groups, N]; final_state: [nb, heads, P, N] fp32, nullable.
constexpr int kSsdMaxState = 128;    // N: a multiple of 16 up to this
constexpr int kSsdMaxHeadDim = 64;   // P: a multiple of 16 up to this (one wave per 16 channels)
constexpr int kSsdThreads = 64 * kSsdMaxHeadDim / 16;  // a workgroup's threads, whatever P
constexpr int kSsdMaxSegments = 16;  // pieces the sequence of one (batch row, head) may be cut into
// How a launch cuts each (batch row, head)'s sequence: `segments` pieces of `seg_chunks` chunks each
// (the last may be shorter). With one segment a workgroup walks the whole sequence and no workspace is
// used; with more, the segments' own state contributions go through the workspace.
struct SsdPlan {
    int64_t segments, seg_chunks;
};
// `split` false: one segment, whatever the shape.
SsdPlan ssd_plan(int64_t nb, int64_t L, int64_t heads, bool io_bf16, bool split);
// State columns the kernels work with: N rounded up to 1, 2, 4 or 8 tiles of 16.
int64_t ssd_state_cols(int64_t N);
// Workspace bytes for a plan (0 for one segment): the segments' decay sums, then their states (rows of
// ssd_state_cols(N) numbers).
size_t ssd_workspace_bytes(const SsdPlan& plan, int64_t nb, int64_t heads, int64_t P, int64_t N);
struct SsdArgs {
    const void* x;
    const float* a;
    const void* b;
    const void* c;
    void* y;
    float* final_state;
    int64_t nb, L, heads, P, N, groups;
    int out_f32;
    SsdPlan plan;
    float* ws_decay;  // [nb, heads, segments]: each segment's sum of a, times log2(e)
    float* ws_state;  // [nb, heads, segments - 1, P, ssd_state_cols(N)]: a segment's state from zero, then the
                      // state entering the next
};
// `workspace` holds ssd_workspace_bytes(plan, ...) bytes (NULL when the plan has one segment).
hipError_t launch_ssd_scan(SsdArgs a, bool io_bf16, void* workspace, hipStream_t stream);

// The device array the entry point that allocates nothing uses as its workspace (noalloc.hip): its
// size, and its address on the current device (looked up once per device; cleared on first use by a
// kernel enqueued on `stream`).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_workspace(hipStream_t stream, void** ws);

}  // namespace ssm
