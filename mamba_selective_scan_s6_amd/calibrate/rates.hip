// rates.hip - calibration kernels for the roofline denominators (gfx950), built as libssmcal.so.
//
// Not part of the selective-scan library: bench.py times these to measure what this device
// sustains, next to the published peaks it reports against:
//   * a plain device copy (HBM read + write bandwidth);
//   * independent fp32 FMA chains with every operand in a VGPR (VALU issue rate);
//   * independent v_exp_f32 chains (transcendental issue rate);
//   * the scan's per-element-step mix: one exponential of a product and three FMA-class operations
//     (decay argument, decay, write, recurrence FMA, readout FMA), exponentials grouped by four.
// Each kernel is launched with a grid the caller chooses; results are written to `out` so that
// nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void copy_kernel(const float4* __restrict__ a, float4* __restrict__ b, int64_t n) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) b[i] = a[i];
}

__device__ __forceinline__ void keep8(float (&a)[8]) {
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7]));
}

// 8 chains x 4 FMAs per iteration per lane
__global__ __launch_bounds__(256) void fma_kernel(float* out, int iters, float s0) {
    float s = s0 + threadIdx.x * 1e-9f, c = 0.25f + threadIdx.x * 1e-9f;
    asm volatile("" : "+v"(s), "+v"(c));
    float a[8];
    for (int i = 0; i < 8; ++i) a[i] = threadIdx.x * 1e-3f + i;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = fmaf(a[i], s, c); a[i] = fmaf(a[i], s, c); a[i] = fmaf(a[i], s, c); a[i] = fmaf(a[i], s, c);
        }
        keep8(a);
    }
    float r = 0.0f;
    for (int i = 0; i < 8; ++i) r += a[i];
    out[blockIdx.x * 256 + threadIdx.x] = r;
}

// 8 chains x 1 exponential per iteration per lane
__global__ __launch_bounds__(256) void exp_kernel(float* out, int iters, float s0) {
    float a[8];
    for (int i = 0; i < 8; ++i) a[i] = -1e-3f * (threadIdx.x + i) * s0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = __builtin_amdgcn_exp2f(a[i]);
        keep8(a);
    }
    float r = 0.0f;
    for (int i = 0; i < 8; ++i) r += a[i];
    out[blockIdx.x * 256 + threadIdx.x] = r;
}

// 16 states per lane, per iteration: decay argument (mul), decay (exp), write (mul), recurrence
// (fma), readout (fma): one element-step of the scan per state
__global__ __launch_bounds__(256) void step_kernel(float* out, int iters, float s0) {
    float s = s0 + threadIdx.x * 1e-9f;
    asm volatile("" : "+v"(s));
    float a2[16], h[16], bq[16], cq[16];
    for (int i = 0; i < 16; ++i) {
        a2[i] = -0.01f * (i + 1);
        h[i] = 0.0f;
        bq[i] = 0.1f * i;
        cq[i] = 0.2f - 0.01f * i;
    }
    float dt = 0.5f + threadIdx.x * 1e-6f, x = 0.3f + threadIdx.x * 1e-6f, acc = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int g = 0; g < 16; g += 4) {
            float e[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) e[k] = __builtin_amdgcn_exp2f(dt * a2[g + k]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                h[g + k] = fmaf(e[k], h[g + k], bq[g + k] * x);
                acc = fmaf(cq[g + k], h[g + k], acc);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        dt = fmaf(dt, s, 1e-5f);
        x = fmaf(x, s, 1e-5f);
        asm volatile("" : "+v"(acc), "+v"(dt), "+v"(x));
    }
    float r = acc;
    for (int i = 0; i < 16; ++i) r += h[i];
    out[blockIdx.x * 256 + threadIdx.x] = r;
}

}  // namespace

extern "C" {

// Copy `bytes` (a multiple of 16) from src to dst on `stream` with `grid` workgroups of 256 threads.
int ssmcal_copy(const void* src, void* dst, int64_t bytes, int grid, void* stream) {
    if (!src || !dst || bytes <= 0 || bytes % 16 || grid < 1) return 1;
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const float4*>(src), static_cast<float4*>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// kind 0: FMA chains (32 FMAs per lane per iteration); 1: exponential chains (8 per lane per
// iteration); 2: the scan's element-step mix (16 element-steps per lane per iteration). `out` holds
// grid * 256 floats.
int ssmcal_rate(int kind, float* out, int iters, int grid, void* stream) {
    if (!out || iters < 1 || grid < 1 || kind < 0 || kind > 2) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (kind == 0) hipLaunchKernelGGL(fma_kernel, dim3(grid), dim3(256), 0, s, out, iters, 0.999f);
    if (kind == 1) hipLaunchKernelGGL(exp_kernel, dim3(grid), dim3(256), 0, s, out, iters, 0.999f);
    if (kind == 2) hipLaunchKernelGGL(step_kernel, dim3(grid), dim3(256), 0, s, out, iters, 0.999f);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
