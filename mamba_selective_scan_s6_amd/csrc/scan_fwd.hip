// scan_fwd.hip - selective scan forward (gfx950).
//
// Computes, per batch row b, channel d and token t ("Beyond attention with Mamba, state space
// models and hybrids", sections 3-4; "Module 19: State-Space Models (Mamba)", The Math):
//   Delta = softplus(delta + bias);  h_n = exp(Delta A_n) h_n + Delta B_{t,n} u;
//   y = sum_n C_{t,n} h_n + D u;  out = y * SiLU(z)
// with the states kept in registers and never written to memory.
//
// Mapping: one wavefront = 64 consecutive channels of one batch row; a lane owns one channel and
// its 16 states. B and C are shared by every channel of a batch row, so each token's rows are
// read with wave-uniform addresses (scalar loads into SGPRs) and feed the VALU directly.
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {
namespace {

template <typename IO, int NFIX>
__global__ __launch_bounds__(64) void scan_seq_kernel(ScanArgs p) {
    using T = typename IO::storage;
    const int lane = threadIdx.x;
    const int64_t groups = (p.nd + 63) / 64;
    const int64_t b = blockIdx.x / groups;
    const int64_t d = (blockIdx.x % groups) * 64 + lane;
    const bool active = d < p.nd;
    const int64_t dc = active ? d : p.nd - 1;  // idle lanes read a valid row and store nothing
    const int N = NFIX == kMaxState ? kMaxState : p.N;
    const int64_t L = p.L;

    float a2[kMaxState];  // A * log2(e): exp(Delta A) = 2^(Delta * a2)
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) a2[n] = n < N ? p.A[dc * N + n] * kLog2e : 0.0f;
    const float bias = p.delta_bias ? p.delta_bias[dc] : 0.0f;
    const float skip = p.D ? p.D[dc] : 0.0f;

    const int64_t row = (b * p.nd + dc) * L;
    const T* __restrict__ u = static_cast<const T*>(p.u) + row;
    const T* __restrict__ dl = static_cast<const T*>(p.delta) + row;
    const T* __restrict__ zz = p.z ? static_cast<const T*>(p.z) + row : nullptr;
    T* __restrict__ out = static_cast<T*>(p.out) + row;
    const T* __restrict__ Bb = static_cast<const T*>(p.B) + b * L * N;
    const T* __restrict__ Cb = static_cast<const T*>(p.C) + b * L * N;

    float h[kMaxState];
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) h[n] = 0.0f;

    for (int64_t t = 0; t < L; ++t) {
        float bv[kMaxState], cv[kMaxState];
        load_row<NFIX>(Bb + t * N, N, bv);
        load_row<NFIX>(Cb + t * N, N, cv);
        const float x = load_elem(u, t);
        const float r = load_elem(dl, t) + bias;
        const float dt = p.softplus ? softplus_f32(r) : r;
        const float dx = dt * x;
        float y = 0.0f;
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) {
            const float abar = exp2_hw(dt * a2[n]);
            h[n] = fmaf(abar, h[n], dx * bv[n]);
            y = fmaf(cv[n], h[n], y);
        }
        y = fmaf(skip, x, y);
        if (zz) y *= silu_f32(load_elem(zz, t));
        if (active) store_elem(out, t, y);
    }
    if (active && p.last_state) {
        float* st = p.last_state + (b * p.nd + d) * N;
#pragma unroll
        for (int n = 0; n < kMaxState; ++n)
            if (n < N) st[n] = h[n];
    }
}

template <typename IO, int NFIX>
hipError_t launch_typed(const ScanArgs& a, hipStream_t s) {
    const int64_t groups = (a.nd + 63) / 64;
    const int64_t blocks = groups * a.nb;
    hipLaunchKernelGGL((scan_seq_kernel<IO, NFIX>), dim3(static_cast<uint32_t>(blocks)), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_fwd(const ScanArgs& a, bool io_bf16, hipStream_t s) {
    if (io_bf16) return a.N == kMaxState ? launch_typed<bf16_io, kMaxState>(a, s) : launch_typed<bf16_io, 0>(a, s);
    return a.N == kMaxState ? launch_typed<f32_io, kMaxState>(a, s) : launch_typed<f32_io, 0>(a, s);
}

}  // namespace ssm
