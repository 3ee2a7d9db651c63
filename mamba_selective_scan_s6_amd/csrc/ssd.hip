// ssd.hip - Mamba-2 scan with a scalar decay per head (gfx950, matrix cores).
//
// For every batch row b and head h, with a state H of P x N numbers that starts at zero
// ("Beyond attention with Mamba, state space models and hybrids", section 8):
//   H_t = exp(a_t) H_{t-1} + x_t b_t^T,   y_t = H_t c_t
// which unrolls to a masked attention, y_t = sum_{s<=t} (c_t . b_s) e^{a_{s+1}+...+a_t} x_s. The
// kernel follows the page's chunked algorithm: the sequence is cut into chunks of kT tokens and, per
// chunk, (1) inside the chunk the scores c_t . b_s are masked by the decay and applied to x; (2) the
// chunk's own contribution to the state is sum_s e^{a_{s+1}+...+a_end} x_s b_s^T; (3) the state
// entering the next chunk is e^{a over the chunk} times the entering state plus that contribution;
// (4) each position reads e^{a_{t0}+...+a_t} c_t from the state entering its chunk.
//
// Mapping. One workgroup per (batch row, head) walks the chunks in order, so the state passes from
// chunk to chunk in registers; its waves split the head's P channels into slices of 16, each wave
// holding its slice of the state (N x 16, fp32) as matrix-core accumulators. Every product is a
// 16 x 16 tile on the matrix cores (v_mfma_f32_16x16x16_bf16 for bf16 inputs, v_mfma_f32_16x16x4_f32
// for fp32 inputs): the chunk's scores are computed transposed (b_s . c_t, a tile per pair of 16-token
// blocks with s <= t), which puts them directly in the operand layout of the next product with x.
// With bf16 inputs the products of the inputs themselves are exact; the fp32 intermediates that feed
// a second product (the masked scores, the state, the decay-weighted x) are split into a bf16 high
// part and a bf16 remainder, two products each, so the result keeps about 16 bits more than one bf16
// rounding would. The chunk's b, c (also b transposed) and x (transposed) are staged in LDS.
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {
namespace {

typedef short sh4 __attribute__((ext_vector_type(4)));
typedef float fl4 __attribute__((ext_vector_type(4)));

template <typename IO>
struct SsdCfg {
    // tokens per chunk: the LDS of a workgroup (at most 64 KB) holds the chunk's b, c, b transposed
    // and x transposed
    static constexpr int kT = IO::bytes == 2 ? 64 : 32;
    // padding per LDS row: rows stay multiples of 16 bytes (aligned 16-byte staging stores and
    // operand reads) and consecutive rows start in different banks
    static constexpr int kPad = 16 / IO::bytes;
};

template <typename IO>
struct SsdLds {
    using E = typename IO::storage;
    static constexpr int kT = SsdCfg<IO>::kT, kPad = SsdCfg<IO>::kPad;
    E b[kT][kSsdMaxState + kPad];    // [token][state]
    E c[kT][kSsdMaxState + kPad];    // [token][state]
    E bt[kSsdMaxState][kT + kPad];   // [state][token]
    E xt[kSsdMaxHeadDim][kT + kPad]; // [channel][token]
    float acum[kT];                  // a_{t0} + ... + a_t, times log2(e)
};

// One lane's operand fragment: 4 consecutive k of a row (A operand) or of a column (B operand),
// bf16 bits or fp32 values.
__device__ __forceinline__ sh4 frag_at(const uint16_t* p) { return *reinterpret_cast<const sh4*>(p); }
__device__ __forceinline__ fl4 frag_at(const float* p) { return *reinterpret_cast<const fl4*>(p); }

// D += A B over 16 k: one bf16 instruction, or four fp32 ones (instruction j takes each lane's j-th k).
__device__ __forceinline__ fl4 mma(sh4 a, sh4 b, fl4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ fl4 mma(fl4 a, fl4 b, fl4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
__device__ __forceinline__ float bf16_value(uint16_t w) { return __uint_as_float(static_cast<uint32_t>(w) << 16); }

// v = hi + lo with hi, lo bf16 (round to nearest each): the error left is about 2^-16 of |v|.
__device__ __forceinline__ void split(fl4 v, sh4& hi, sh4& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint16_t h = bf16_bits(v[i]);
        hi[i] = static_cast<short>(h);
        lo[i] = static_cast<short>(bf16_bits(v[i] - bf16_value(h)));
    }
}

// D += A B where A (fa) or B (fb) holds fp32 values and the other operand is an input fragment.
__device__ __forceinline__ fl4 mma_fa(fl4 a, sh4 b, fl4 c) {
    sh4 hi, lo;
    split(a, hi, lo);
    return mma(lo, b, mma(hi, b, c));
}
__device__ __forceinline__ fl4 mma_fa(fl4 a, fl4 b, fl4 c) { return mma(a, b, c); }
__device__ __forceinline__ fl4 mma_fb(sh4 a, fl4 b, fl4 c) {
    sh4 hi, lo;
    split(b, hi, lo);
    return mma(a, lo, mma(a, hi, c));
}
__device__ __forceinline__ fl4 mma_fb(fl4 a, fl4 b, fl4 c) { return mma(a, b, c); }

// Eight consecutive elements of a global row (zeros when the row lies past the end), as stored.
template <typename E>
struct Oct;
template <>
struct Oct<uint16_t> {
    uint4 v;
    __device__ __forceinline__ void load(const uint16_t* p, bool in) { v = in ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ uint16_t get(int i) const {
        const uint32_t w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
        return static_cast<uint16_t>((i & 1) ? (w >> 16) : (w & 0xffffu));
    }
    __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<uint4*>(p) = v; }
};
template <>
struct Oct<float> {
    float4 v0, v1;
    __device__ __forceinline__ void load(const float* p, bool in) {
        if (in) {
            v0 = reinterpret_cast<const float4*>(p)[0];
            v1 = reinterpret_cast<const float4*>(p)[1];
        } else {
            v0 = v1 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }
    __device__ __forceinline__ float get(int i) const {
        const float4& q = i < 4 ? v0 : v1;
        const int k = i & 3;
        return k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w;
    }
    __device__ __forceinline__ void store(float* p) const {
        reinterpret_cast<float4*>(p)[0] = v0;
        reinterpret_cast<float4*>(p)[1] = v1;
    }
};

template <typename OT>
__device__ __forceinline__ void store_out(OT* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float v) { *p = bf16_bits(v); }

template <typename IO>
__device__ __forceinline__ float as_float(typename IO::storage e) {
    if constexpr (IO::bytes == 2) return bf16_value(e);
    else return e;
}

template <typename IO, typename OT>
__global__ __launch_bounds__(64 * kSsdMaxHeadDim / 16) void ssd_kernel(SsdArgs p) {
    using E = typename IO::storage;
    constexpr int kT = SsdCfg<IO>::kT;
    constexpr int kTT = kT / 16;  // 16-token blocks per chunk
    __shared__ __align__(16) SsdLds<IO> s;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, k4 = 4 * (lane >> 4);  // operand row / column, and first of 4 k
    const int nthreads = blockDim.x;
    const int64_t H = p.heads, P = p.P, N = p.N, G = p.groups, L = p.L;
    const int64_t bi = blockIdx.x / H, h = blockIdx.x - bi * H;
    const int64_t g = h / (H / G);
    const int p0 = 16 * wave;  // this wave's slice of the head's channels
    const int ntile = static_cast<int>(N / 16);
    const E* __restrict__ xg = static_cast<const E*>(p.x);
    const E* __restrict__ bg = static_cast<const E*>(p.b);
    const E* __restrict__ cg = static_cast<const E*>(p.c);

    fl4 z[kSsdMaxState / 16];  // the state's slice: z[nt][i] = H[p0 + r16][16 nt + k4 + i] (rows n, columns p)
#pragma unroll
    for (int nt = 0; nt < kSsdMaxState / 16; ++nt) z[nt] = fl4{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t nchunks = (L + kT - 1) / kT;
    for (int64_t ck = 0; ck < nchunks; ++ck) {
        const int64_t t0 = ck * kT;
        // ---- stage the chunk: b, c (and b transposed) by token rows, x transposed, the cumulative decay
        for (int e = threadIdx.x * 8; e < kT * N; e += nthreads * 8) {
            const int t = e / static_cast<int>(N), n = e - t * static_cast<int>(N);
            const bool in = t0 + t < L;
            const int64_t off = ((bi * L + t0 + t) * G + g) * N + n;
            Oct<E> vb, vc;
            vb.load(bg + off, in);
            vc.load(cg + off, in);
            vb.store(&s.b[t][n]);
            vc.store(&s.c[t][n]);
#pragma unroll
            for (int i = 0; i < 8; ++i) s.bt[n + i][t] = vb.get(i);
        }
        for (int e = threadIdx.x * 8; e < kT * P; e += nthreads * 8) {
            const int t = e / static_cast<int>(P), q = e - t * static_cast<int>(P);
            const bool in = t0 + t < L;
            Oct<E> vx;
            vx.load(xg + ((bi * L + t0 + t) * H + h) * P + q, in);
#pragma unroll
            for (int i = 0; i < 8; ++i) s.xt[q + i][t] = vx.get(i);
        }
        if (wave == 0 && lane < kT) {
            // inclusive prefix sum of a over the chunk (0 past the end: the state then stays as it is)
            float v = t0 + lane < L ? p.a[(bi * L + t0 + lane) * H + h] * kLog2e : 0.0f;
#pragma unroll
            for (int d = 1; d < kT; d *= 2) {
                const float o = __shfl_up(v, d, 64);
                if (lane >= d) v += o;
            }
            s.acum[lane] = v;
        }
        __syncthreads();

        // ---- outputs of the chunk, one 16-token block at a time
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt) {
            fl4 yin = {0.0f, 0.0f, 0.0f, 0.0f};
            const float at = s.acum[16 * tt + r16];  // row t of the transposed score tiles
#pragma unroll
            for (int st = 0; st <= tt; ++st) {
                // scores, transposed: gt[i] = b_s . c_t with s = 16 st + k4 + i, t = 16 tt + r16
                fl4 gt = {0.0f, 0.0f, 0.0f, 0.0f};
                for (int kb = 0; kb < ntile; ++kb)
                    gt = mma(frag_at(&s.b[16 * st + r16][16 * kb + k4]), frag_at(&s.c[16 * tt + r16][16 * kb + k4]), gt);
                // masked by the decay between s and t: the A operand of the product with x (row t, k s)
                fl4 m;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int sl = 16 * st + k4 + i, tl = 16 * tt + r16;
                    m[i] = sl <= tl ? gt[i] * exp2_hw(at - s.acum[sl]) : 0.0f;
                }
                yin = mma_fa(m, frag_at(&s.xt[p0 + r16][16 * st + k4]), yin);
            }
            // what the block's tokens read from the state entering the chunk
            fl4 yen = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int nt = 0; nt < ntile; ++nt) yen = mma_fb(frag_at(&s.c[16 * tt + r16][16 * nt + k4]), z[nt], yen);
            // yin, yen: rows t = 16 tt + k4 + i, column p = p0 + r16
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tl = 16 * tt + k4 + i;
                const int64_t t = t0 + tl;
                if (t < L) {
                    const float y = fmaf(exp2_hw(s.acum[tl]), yen[i], yin[i]);
                    store_out(static_cast<OT*>(p.y) + ((bi * L + t) * H + h) * P + p0 + r16, y);
                }
            }
        }

        // ---- the state leaving the chunk: decayed over the chunk, plus sum_s e^{a_{s+1}..a_end} x_s b_s^T
        {
            const float aend = s.acum[kT - 1];
            fl4 wxv[kTT];
#pragma unroll
            for (int sb = 0; sb < kTT; ++sb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int sl = 16 * sb + k4 + i;
                    wxv[sb][i] = exp2_hw(aend - s.acum[sl]) * as_float<IO>(s.xt[p0 + r16][sl]);
                }
            }
            const float dend = exp2_hw(aend);
            for (int nt = 0; nt < ntile; ++nt) {
                fl4 acc = z[nt] * dend;
#pragma unroll
                for (int sb = 0; sb < kTT; ++sb) acc = mma_fb(frag_at(&s.bt[16 * nt + r16][16 * sb + k4]), wxv[sb], acc);
                z[nt] = acc;
            }
        }
        __syncthreads();  // every wave is done with the chunk's LDS before the next is staged
    }

    if (p.final_state) {
        float* fs = p.final_state + ((bi * H + h) * P + p0 + r16) * N;
        for (int nt = 0; nt < ntile; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) fs[16 * nt + k4 + i] = z[nt][i];
    }
}

template <typename IO, typename OT>
hipError_t launch_ssd_typed(const SsdArgs& a, hipStream_t st) {
    const uint32_t blocks = static_cast<uint32_t>(a.nb * a.heads);
    hipLaunchKernelGGL((ssd_kernel<IO, OT>), dim3(blocks), dim3(static_cast<uint32_t>(64 * (a.P / 16))), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ssd_scan(const SsdArgs& a, bool io_bf16, hipStream_t st) {
    if (!io_bf16) return launch_ssd_typed<f32_io, float>(a, st);
    return a.out_f32 ? launch_ssd_typed<bf16_io, float>(a, st) : launch_ssd_typed<bf16_io, uint16_t>(a, st);
}

}  // namespace ssm
