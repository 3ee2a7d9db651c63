// conv1d.hip - causal depthwise convolution + SiLU, and its one-token window update (gfx950).
//
// The step just before the selective scan in the Mamba block ("Module 19: State-Space Models
// (Mamba)", The Causal Convolution and The Math: Six Stages; "Beyond attention with Mamba, state
// space models and hybrids", section 4, the Mixer's conv1d, and section 7, mixer_step's window):
//   u[b,d,t] = act(bias[d] + sum_{k<K} w[d,k] x[b,d,t-(K-1)+k]),  x at t < 0 read as 0,
// with act = SiLU (or the identity). Each channel has its own K taps; channels never mix.
//
// The scan's steps, B and C come from u through a projection, so u is written to memory here and
// the scan reads it like any other input (folding this into the scan's load would read x instead
// of u: the same bytes).
//
// Mapping (sequence): a lane owns 8 or 16 consecutive tokens of one channel row; consecutive lanes take
// consecutive chunks of a row, so the 16-byte vector loads and stores of a wave are contiguous.
// The K-1 inputs before a chunk are shuffled in from the lane to the left. Bound by memory: each
// input and output element is touched once.
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {
namespace {

constexpr int kThreadsConv = 256;
// Tokens per lane: 16 on large problems (two 16-byte loads in flight per lane), 8 where that would
// leave too few waves to fill the GPU (measured: 45 vs 56 us on 4 x 5120 x 2048 bf16; 8.2 vs 9.9 us
// on 1 x 1536 x 2048 fp32).
constexpr int64_t kLongChunkElems = int64_t(8) << 20;

// KF: the convolution width when fixed at compile time (0: taken from the arguments). With a fixed width
// every tap's index into the lane's inputs is a constant; with a runtime width each one is selected from
// the possible positions, which cost ~20% of the kernel's time on large shapes.
template <typename IO, bool SILU, bool VEC, int kChunk, int KF>
__global__ __launch_bounds__(kThreadsConv) void causal_conv1d_kernel(ConvArgs p) {
    static_assert(kChunk % 8 == 0 && kChunk >= kMaxConvWidth - 1, "chunk: a multiple of 8 covering the halo");
    using T = typename IO::storage;
    const int64_t chunks = (p.L + kChunk - 1) / kChunk;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreadsConv + threadIdx.x;
    if (gid >= p.nb * p.nd * chunks) return;
    const int64_t row = gid / chunks;  // b * nd + d
    const int64_t t0 = (gid - row * chunks) * kChunk;
    const int64_t d = row % p.nd;
    const int K = KF > 0 ? KF : p.K;
    const T* __restrict__ xr = static_cast<const T*>(p.x) + row * p.L;

    float w[kMaxConvWidth];
#pragma unroll
    for (int k = 0; k < kMaxConvWidth; ++k) w[k] = k < K ? p.w[d * K + k] : 0.0f;
    const float bias = p.bias ? p.bias[d] : 0.0f;

    // v[i] = x[t0 - (kMaxConvWidth - 1) + i], i < kMaxConvWidth - 1 + kChunk (zeros outside [0, L))
    constexpr int kHalo = kMaxConvWidth - 1;
    float v[kHalo + kChunk];
    // The K-1 inputs before the chunk, from memory, loaded together with the chunk and used only where
    // the left lane cannot supply them: a load issued after the chunk's values are used (the shuffle
    // below) would cost its lanes a second memory round trip. With VEC the 8 inputs before the chunk are
    // one 16-byte vector (two with fp32); a row's first chunk reads its own start instead (dropped).
    static_assert(kHalo <= 8 && kChunk % 8 == 0, "the halo fits the 8 elements before the chunk");
    float hmem[kHalo];
    if (VEC) {
        const int64_t th = t0 >= 8 ? t0 - 8 : 0;
        float e[8];
        if constexpr (IO::bytes == 4) {
            const float4* q = reinterpret_cast<const float4*>(xr + th);
            const float4 a = q[0], b = q[1];
            e[0] = a.x; e[1] = a.y; e[2] = a.z; e[3] = a.w; e[4] = b.x; e[5] = b.y; e[6] = b.z; e[7] = b.w;
        } else {
            const uint4 q = *reinterpret_cast<const uint4*>(xr + th);
            e[0] = bf16_lo(q.x); e[1] = bf16_hi(q.x); e[2] = bf16_lo(q.y); e[3] = bf16_hi(q.y);
            e[4] = bf16_lo(q.z); e[5] = bf16_hi(q.z); e[6] = bf16_lo(q.w); e[7] = bf16_hi(q.w);
        }
#pragma unroll
        for (int i = 0; i < kHalo; ++i) hmem[i] = e[8 - kHalo + i];
    } else {
#pragma unroll
        for (int i = 0; i < kHalo; ++i) {
            const int64_t t = t0 - kHalo + i;
            hmem[i] = i >= kHalo - (K - 1) ? load_elem(xr, t >= 0 ? t : 0) : 0.0f;
        }
    }
    if (VEC && t0 + kChunk <= p.L) {
#pragma unroll
        for (int c = 0; c < kChunk; c += 8) {
            float* dst = v + kHalo + c;
            if constexpr (IO::bytes == 4) {
                const float4* q = reinterpret_cast<const float4*>(xr + t0 + c);
                const float4 a = q[0], b = q[1];
                dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
                dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
            } else {
                const uint4 q = *reinterpret_cast<const uint4*>(xr + t0 + c);
                dst[0] = bf16_lo(q.x); dst[1] = bf16_hi(q.x); dst[2] = bf16_lo(q.y); dst[3] = bf16_hi(q.y);
                dst[4] = bf16_lo(q.z); dst[5] = bf16_hi(q.z); dst[6] = bf16_lo(q.w); dst[7] = bf16_hi(q.w);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kChunk; ++j) v[kHalo + j] = t0 + j < p.L ? load_elem(xr, t0 + j) : 0.0f;
    }

    // The K-1 inputs before the chunk are the last ones of the lane to the left when it holds the
    // previous chunk of the same row (a shuffle); a wave's first lane and a row's first chunk read
    // them from memory (zeros before t = 0).
    const int lane = threadIdx.x & 63;
    const bool left_has_them = lane != 0 && t0 != 0;
#pragma unroll
    for (int i = 0; i < kHalo; ++i) {
        const float from_left = __shfl_up(v[kHalo + kChunk - kHalo + i], 1);
        if (i >= kHalo - (K - 1)) {
            const int64_t t = t0 - kHalo + i;
            v[i] = left_has_them ? from_left : (t >= 0 ? hmem[i] : 0.0f);
        } else {
            v[i] = 0.0f;
        }
    }

    float o[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
        // output t0 + j reads inputs t0 + j - (K-1) .. t0 + j, i.e. v[kHalo + j - (K-1) + k]
        float pre = bias;
#pragma unroll
        for (int k = 0; k < kMaxConvWidth; ++k)
            if (k < K) pre = fmaf(w[k], v[kHalo + j - (K - 1) + k], pre);
        o[j] = SILU ? silu_f32(pre) : pre;
    }

    T* __restrict__ orow = static_cast<T*>(p.out) + row * p.L;
    if (VEC && t0 + kChunk <= p.L) {
#pragma unroll
        for (int c = 0; c < kChunk; c += 8) {
            const float* src = o + c;
            if constexpr (IO::bytes == 4) {
                float4* q = reinterpret_cast<float4*>(orow + t0 + c);
                q[0] = make_float4(src[0], src[1], src[2], src[3]);
                q[1] = make_float4(src[4], src[5], src[6], src[7]);
            } else {
                uint32_t wd[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(src[2 * k]));
                    const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(src[2 * k + 1]));
                    wd[k] = lo | (hi << 16);
                }
                *reinterpret_cast<uint4*>(orow + t0 + c) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kChunk; ++j)
            if (t0 + j < p.L) store_elem(orow, t0 + j, o[j]);
    }
}

// One decode step: window[b,d,:] <- (window[b,d,1:], x[b,d]); out = act(bias + taps . window).
template <typename IO, bool SILU>
__global__ __launch_bounds__(kThreadsConv) void conv_window_kernel(ConvArgs p) {
    using T = typename IO::storage;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kThreadsConv + threadIdx.x;
    if (row >= p.nb * p.nd) return;
    const int64_t d = row % p.nd;
    const int K = p.K;
    float* win = p.window + row * K;
    float v[kMaxConvWidth];
#pragma unroll
    for (int k = 0; k + 1 < kMaxConvWidth; ++k) v[k] = k + 1 < K ? win[k + 1] : 0.0f;
    const float xn = load_elem(static_cast<const T*>(p.x), row);
    float pre = p.bias ? p.bias[d] : 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxConvWidth; ++k) {
        if (k + 1 < K) {
            pre = fmaf(p.w[d * K + k], v[k], pre);
            win[k] = v[k];
        } else if (k + 1 == K) {
            pre = fmaf(p.w[d * K + k], xn, pre);
            win[k] = xn;
        }
    }
    store_elem(static_cast<T*>(p.out), row, SILU ? silu_f32(pre) : pre);
}

template <typename IO, bool SILU, int kChunk, int KF>
hipError_t launch_conv_chunk(const ConvArgs& a, hipStream_t s) {
    const int64_t chunks = (a.L + kChunk - 1) / kChunk;
    const int64_t blocks = (a.nb * a.nd * chunks + kThreadsConv - 1) / kThreadsConv;
    // 16-byte vectors: rows a multiple of 16 bytes long, and at least 8 elements (the halo vector of a
    // row's first chunk reads elements 0..7)
    if (a.L % (16 / IO::bytes) == 0 && a.L >= 8)
        hipLaunchKernelGGL((causal_conv1d_kernel<IO, SILU, true, kChunk, KF>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(kThreadsConv), 0, s, a);
    else
        hipLaunchKernelGGL((causal_conv1d_kernel<IO, SILU, false, kChunk, KF>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(kThreadsConv), 0, s, a);
    return hipGetLastError();
}

template <typename IO, bool SILU, int kChunk>
hipError_t launch_conv_width(const ConvArgs& a, hipStream_t s) {
    switch (a.K) {  // the widths Mamba layers use get kernels of their own
        case 2: return launch_conv_chunk<IO, SILU, kChunk, 2>(a, s);
        case 3: return launch_conv_chunk<IO, SILU, kChunk, 3>(a, s);
        case 4: return launch_conv_chunk<IO, SILU, kChunk, 4>(a, s);
        default: return launch_conv_chunk<IO, SILU, kChunk, 0>(a, s);
    }
}

template <typename IO, bool SILU>
hipError_t launch_conv_typed(const ConvArgs& a, hipStream_t s) {
    if (a.nb * a.nd * a.L >= kLongChunkElems) return launch_conv_width<IO, SILU, 16>(a, s);
    return launch_conv_width<IO, SILU, 8>(a, s);
}

template <typename IO, bool SILU>
hipError_t launch_window_typed(const ConvArgs& a, hipStream_t s) {
    const int64_t blocks = (a.nb * a.nd + kThreadsConv - 1) / kThreadsConv;
    hipLaunchKernelGGL((conv_window_kernel<IO, SILU>), dim3(static_cast<uint32_t>(blocks)), dim3(kThreadsConv), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int64_t conv_max_blocks(int64_t nb, int64_t nd, int64_t L) {
    return ceil_div(sat_mul(sat_mul(nb, nd), ceil_div(L, 8)), kThreadsConv);  // at 8 tokens per lane (the most)
}

hipError_t launch_causal_conv1d(const ConvArgs& a, bool io_bf16, hipStream_t s) {
    if (io_bf16) return a.silu ? launch_conv_typed<bf16_io, true>(a, s) : launch_conv_typed<bf16_io, false>(a, s);
    return a.silu ? launch_conv_typed<f32_io, true>(a, s) : launch_conv_typed<f32_io, false>(a, s);
}

hipError_t launch_conv_window_update(const ConvArgs& a, bool io_bf16, hipStream_t s) {
    if (io_bf16) return a.silu ? launch_window_typed<bf16_io, true>(a, s) : launch_window_typed<bf16_io, false>(a, s);
    return a.silu ? launch_window_typed<f32_io, true>(a, s) : launch_window_typed<f32_io, false>(a, s);
}

}  // namespace ssm
