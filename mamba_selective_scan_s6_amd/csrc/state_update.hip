// state_update.hip - one-token decode update of the selective-scan state (gfx950).
//
// The recurrence of the scan for a single position with the state carried by the caller
// ("Beyond attention with Mamba, state space models and hybrids", section 7, mixer_step):
//   Delta = softplus(delta);  h_n <- exp(Delta A_n) h_n + Delta B_n x;
//   y = sum_n C_n h_n + D x;  out = y * SiLU(z)
// The state [batch, dim, N] fp32 is read and written in place: this path is bound by memory
// bandwidth, 128 bytes of state traffic per channel against 16 exponentials.
//
// Mapping: one wavefront = 64 consecutive channels of one batch row, a lane per channel with its
// 16 states in registers; B and C of the batch row are wave-uniform (scalar loads).
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {
namespace {

template <typename IO, int NFIX>
__global__ __launch_bounds__(64) void state_update_kernel(UpdateArgs p) {
    using T = typename IO::storage;
    const int lane = threadIdx.x;
    const int64_t groups = (p.nd + 63) / 64;
    const int64_t b = blockIdx.x / groups;
    const int64_t d = (blockIdx.x % groups) * 64 + lane;
    if (d >= p.nd) return;
    const int N = NFIX == kMaxState ? kMaxState : p.N;
    const int64_t rowi = b * p.nd + d;

    float bv[kMaxState], cv[kMaxState];
    load_row<NFIX>(static_cast<const T*>(p.B) + b * N, N, bv);
    load_row<NFIX>(static_cast<const T*>(p.C) + b * N, N, cv);

    float h[kMaxState];
    float* st = p.state + rowi * N;
    if constexpr (NFIX == kMaxState) {
        const float4* s4 = reinterpret_cast<const float4*>(st);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 v = s4[k];
            h[4 * k] = v.x; h[4 * k + 1] = v.y; h[4 * k + 2] = v.z; h[4 * k + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) h[n] = n < N ? st[n] : 0.0f;
    }

    const float x = load_elem(static_cast<const T*>(p.x), rowi);
    const float dt = softplus_f32(load_elem(static_cast<const T*>(p.delta), rowi));
    const float dx = dt * x;
    float y = 0.0f;
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) {
        const float a2 = n < N ? p.A[d * N + n] * kLog2e : 0.0f;
        h[n] = fmaf(exp2_hw(dt * a2), h[n], dx * bv[n]);
        y = fmaf(cv[n], h[n], y);
    }
    if (p.D) y = fmaf(p.D[d], x, y);
    if (p.z) y *= silu_f32(load_elem(static_cast<const T*>(p.z), rowi));
    store_elem(static_cast<T*>(p.out), rowi, y);

    if constexpr (NFIX == kMaxState) {
        float4* s4 = reinterpret_cast<float4*>(st);
#pragma unroll
        for (int k = 0; k < 4; ++k) s4[k] = make_float4(h[4 * k], h[4 * k + 1], h[4 * k + 2], h[4 * k + 3]);
    } else {
#pragma unroll
        for (int n = 0; n < kMaxState; ++n)
            if (n < N) st[n] = h[n];
    }
}

template <typename IO, int NFIX>
hipError_t launch_typed(const UpdateArgs& a, hipStream_t s) {
    const int64_t blocks = (a.nd + 63) / 64 * a.nb;
    hipLaunchKernelGGL((state_update_kernel<IO, NFIX>), dim3(static_cast<uint32_t>(blocks)), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state_update(const UpdateArgs& a, bool io_bf16, hipStream_t s) {
    if (io_bf16) return a.N == kMaxState ? launch_typed<bf16_io, kMaxState>(a, s) : launch_typed<bf16_io, 0>(a, s);
    return a.N == kMaxState ? launch_typed<f32_io, kMaxState>(a, s) : launch_typed<f32_io, 0>(a, s);
}

}  // namespace ssm
