// ssm_kernels.hpp - launch interface between the C ABI shim and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
};

// io_bf16: false = fp32 io tensors, true = bf16 io tensors. Arguments are validated by the caller.
hipError_t launch_scan_fwd(const ScanArgs& a, bool io_bf16, hipStream_t stream);
hipError_t launch_state_update(const UpdateArgs& a, bool io_bf16, hipStream_t stream);

}  // namespace ssm
