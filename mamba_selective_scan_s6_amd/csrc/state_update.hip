// state_update.hip - one-token decode update of the selective-scan state (gfx950).
//
// The recurrence of the scan for a single position with the state carried by the caller
// ("Beyond attention with Mamba, state space models and hybrids", section 7, mixer_step):
//   Delta = softplus(delta);  h_n <- exp(Delta A_n) h_n + Delta B_n x;
//   y = sum_n C_n h_n + D x;  out = y * SiLU(z)
// The state [batch, dim, N] fp32 is read and written in place: this path is bound by memory
// bandwidth, 128 bytes of state traffic per channel against 16 exponentials.
//
// Mapping: a workgroup of 256 threads covers 64 consecutive channels of kRows batch rows; four
// consecutive lanes share a channel and each holds 4 of its 16 states. Every state, A, B and C
// access is then one 16-byte (bf16: 8-byte) vector per lane, contiguous across the wave, and the
// readout is summed over the 4 lanes with two xor shuffles (the same order in every lane). All
// loads of the kRows rows are issued before any arithmetic. The kernel is bound by memory: on the
// 64 x 8192 x 16 decode shape it moves the state at the rate of a plain device copy. 2 rows per
// workgroup measured best of 1, 2, 4 and 8.
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {
namespace {

constexpr int kChannels = 64;          // channels per workgroup
constexpr int kLanesPerChannel = 4;    // 4 states per lane
constexpr int kThreads = kChannels * kLanesPerChannel;
constexpr int kRows = 2;               // batch rows per workgroup (their loads are issued together)

// Four consecutive elements of a B or C row starting at n0 (fp32: one 16-byte load; bf16: 8 bytes).
template <typename IO>
__device__ __forceinline__ void load4(const typename IO::storage* __restrict__ p, float (&v)[4]) {
    if constexpr (IO::bytes == 4) {
        const float4 q = *reinterpret_cast<const float4*>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
        const uint2 q = *reinterpret_cast<const uint2*>(p);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    }
}

template <typename IO, int NFIX, bool ZOH>
__global__ __launch_bounds__(kThreads) void state_update_kernel(UpdateArgs p) {
    using T = typename IO::storage;
    const int q = threadIdx.x & (kLanesPerChannel - 1);  // which 4 states
    const int64_t groups = (p.nd + kChannels - 1) / kChannels;
    const int64_t b0 = blockIdx.x / groups * kRows;
    const int64_t d = (blockIdx.x % groups) * kChannels + (threadIdx.x >> 2);
    const bool active = d < p.nd;
    const int64_t dc = active ? d : p.nd - 1;  // idle lanes still take part in the shuffles
    const int N = NFIX == kMaxState ? kMaxState : p.N;
    const int n0 = 4 * q;

    // ---- every load of the kRows rows first, so that they are all in flight together
    const T* zsrc = static_cast<const T*>(p.z ? p.z : p.x);
    float a2[4];
    float bv[kRows][4], cv[kRows][4], h[kRows][4], xr[kRows], rr[kRows], zr[kRows];
    if constexpr (NFIX == kMaxState) {
        const float4 av = *reinterpret_cast<const float4*>(p.A + dc * N + n0);
        a2[0] = av.x * kLog2e; a2[1] = av.y * kLog2e; a2[2] = av.z * kLog2e; a2[3] = av.w * kLog2e;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) a2[i] = n0 + i < N ? p.A[dc * N + n0 + i] * kLog2e : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int64_t b = b0 + r < p.nb ? b0 + r : p.nb - 1;  // rows past the batch: recomputed, not stored
        const int64_t rowi = b * p.nd + dc;
        const float* st = p.state + rowi * N + n0;
        if constexpr (NFIX == kMaxState) {
            load4<IO>(static_cast<const T*>(p.B) + b * N + n0, bv[r]);
            load4<IO>(static_cast<const T*>(p.C) + b * N + n0, cv[r]);
            const float4 sv = *reinterpret_cast<const float4*>(st);
            h[r][0] = sv.x; h[r][1] = sv.y; h[r][2] = sv.z; h[r][3] = sv.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool in = n0 + i < N;
                bv[r][i] = in ? load_elem(static_cast<const T*>(p.B), b * N + n0 + i) : 0.0f;
                cv[r][i] = in ? load_elem(static_cast<const T*>(p.C), b * N + n0 + i) : 0.0f;
                h[r][i] = in ? st[i] : 0.0f;
            }
        }
        xr[r] = load_elem(static_cast<const T*>(p.x), rowi);
        rr[r] = load_elem(static_cast<const T*>(p.delta), rowi);
        // the gate's load is unconditional (x's row stands in when there is no gate; the value is then
        // dropped): a load behind a branch makes the compiler wait for every load issued before it
        const float zv = load_elem(zsrc, rowi);
        zr[r] = p.z ? zv : 0.0f;
    }
    const float skip = p.D ? p.D[dc] : 0.0f;
    float ia[4];  // 1 / A for the zero-order-hold gain
#pragma unroll
    for (int i = 0; i < 4; ++i) ia[i] = ZOH && a2[i] != 0.0f ? kLog2e / a2[i] : 0.0f;

    // ---- update, readout, stores
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int64_t b = b0 + r;
        const float dt = softplus_f32(rr[r]);
        const float dx = dt * xr[r];
        float y = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float yi = dt * a2[i], ai = exp2_hw(yi);
            const float gain = ZOH ? zoh_gain(yi, ai, dt, ia[i]) * xr[r] : dx;
            h[r][i] = fmaf(ai, h[r][i], gain * bv[r][i]);
            y = fmaf(cv[r][i], h[r][i], y);
        }
        // sum over the channel's 4 lanes: (y0 + y1) + (y2 + y3) in every lane of the quad
        y += __shfl_xor(y, 1);
        y += __shfl_xor(y, 2);
        if (active && b < p.nb) {
            const int64_t rowi = b * p.nd + d;
            float* st = p.state + rowi * N + n0;
            if constexpr (NFIX == kMaxState) {
                *reinterpret_cast<float4*>(st) = make_float4(h[r][0], h[r][1], h[r][2], h[r][3]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (n0 + i < N) st[i] = h[r][i];
            }
            if (q == 0) {
                if (p.D) y = fmaf(skip, xr[r], y);
                if (p.z) y *= silu_f32(zr[r]);
                if (p.out_f32) static_cast<float*>(p.out)[rowi] = y;
                else store_elem(static_cast<T*>(p.out), rowi, y);
            }
        }
    }
}

template <typename IO, int NFIX, bool ZOH>
hipError_t launch_typed(const UpdateArgs& a, hipStream_t s) {
    const int64_t blocks = (a.nd + kChannels - 1) / kChannels * ((a.nb + kRows - 1) / kRows);
    hipLaunchKernelGGL((state_update_kernel<IO, NFIX, ZOH>), dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename IO, int NFIX>
hipError_t launch_zoh(const UpdateArgs& a, hipStream_t s) {
    return a.zoh ? launch_typed<IO, NFIX, true>(a, s) : launch_typed<IO, NFIX, false>(a, s);
}

}  // namespace

hipError_t launch_state_update(const UpdateArgs& a, bool io_bf16, hipStream_t s) {
    if (io_bf16) return a.N == kMaxState ? launch_zoh<bf16_io, kMaxState>(a, s) : launch_zoh<bf16_io, 0>(a, s);
    return a.N == kMaxState ? launch_zoh<f32_io, kMaxState>(a, s) : launch_zoh<f32_io, 0>(a, s);
}

}  // namespace ssm
