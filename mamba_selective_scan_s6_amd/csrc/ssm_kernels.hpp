// ssm_kernels.hpp - launch interface between the C ABI shim and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <functional>

namespace ssm {

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
    float* hblk = nullptr;  // optional: state entering each 16-token block, [nb, nd, ceil(L/16), 16]
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
    float* lam = nullptr;    // [nb, nd, nblk, 16] block's reverse aggregate from a zero carry
    float* sdt = nullptr;    // [nb, nd, nblk] block's sum of steps
    float* muin = nullptr;   // [nb, nd, nblk, 16] adjoint carry into each block from the right
    float* dBp = nullptr;    // [groups, nb, L, 16] dB partials per 64-channel group
    float* dCp = nullptr;    // [groups, nb, L, 16]
    float* dAp = nullptr;    // [nb, nseg, nd, 16] dA partials per 64-token segment
    float* dDp = nullptr;    // [nb, nseg, nd]
    float* dbp = nullptr;    // [nb, nseg, nd]
    int64_t groups = 0, nbg = 0, nblk = 0, nseg = 0;
};

// Extra workspace bytes of a backward call (beyond scan_workspace_bytes), and the launch: the
// forward in checkpoint mode on `scan_workspace` (with `epoch`), then the backward kernels on `extra`.
size_t scan_bwd_extra_bytes(int64_t nb, int64_t nd, int64_t L);
hipError_t launch_scan_bwd(BwdArgs q, bool io_bf16, void* scan_workspace, uint32_t epoch, void* extra,
                           hipStream_t stream);

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

// Bytes reserved at the start of a scan workspace (word 0: sticky error flags set by kernels).
constexpr size_t kWorkspaceHeader = 256;

// Scan workspace size for a problem, and the number of workgroups one launch uses.
size_t scan_workspace_bytes(int64_t nb, int64_t nd, int64_t L);
int64_t scan_max_blocks(int64_t nb, int64_t nd, int64_t L);
// Tokens per workgroup segment that launch_scan_fwd uses for this shape.
int scan_segment_tokens(int64_t nb, int64_t nd, int64_t L);

// io_bf16: false = fp32 io tensors, true = bf16 io tensors. Arguments are validated by the caller.
// workspace: scan_workspace_bytes() device bytes, zeroed when first allocated; epoch: a value not
// used by an earlier launch on the same workspace since it was zeroed (1 .. 2^30 - 1).
hipError_t launch_scan_fwd(const ScanArgs& a, bool io_bf16, void* workspace, uint32_t epoch, hipStream_t stream);
// Polls a scan's look-back may wait before recording a timeout (<= 0: the default); returns the previous.
int set_scan_wait_limit(int polls);
hipError_t launch_state_update(const UpdateArgs& a, bool io_bf16, hipStream_t stream);

// Workspace cache, one per (device, stream): see workspace.cpp. Calls launch(workspace, epoch)
// with a workspace of at least `bytes` and a fresh epoch, holding the cache lock.
hipError_t with_scan_workspace(hipStream_t stream, size_t bytes,
                               const std::function<hipError_t(void*, uint32_t)>& launch);
// Synchronise the stream; then report and clear the error flags of its workspace (0 if none).
hipError_t take_workspace_errors(hipStream_t stream, uint32_t* flags);
hipError_t release_workspaces();

}  // namespace ssm
