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
    E x[kT][kSsdMaxHeadDim + kPad];  // [token][channel]
    float acum[kT];                  // a_{t0} + ... + a_t, times log2(e)
};

// One lane's operand fragment: 4 consecutive k of a row (A operand) or of a column (B operand),
// bf16 bits or fp32 values.
__device__ __forceinline__ sh4 frag_at(const uint16_t* p) { return *reinterpret_cast<const sh4*>(p); }
__device__ __forceinline__ fl4 frag_at(const float* p) { return *reinterpret_cast<const fl4*>(p); }
// The same from 4 consecutive rows of one column (row stride `ld` elements).
__device__ __forceinline__ sh4 frag_col(const uint16_t* p, int ld) {
    return sh4{static_cast<short>(p[0]), static_cast<short>(p[ld]), static_cast<short>(p[2 * ld]), static_cast<short>(p[3 * ld])};
}
__device__ __forceinline__ fl4 frag_col(const float* p, int ld) { return fl4{p[0], p[ld], p[2 * ld], p[3 * ld]}; }

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

// An fp32 operand split once for several products: bf16 (hi, lo) with bf16 inputs, the value itself
// with fp32 inputs.
template <typename IO>
struct SplitOp;
template <>
struct SplitOp<bf16_io> {
    sh4 hi, lo;
    __device__ __forceinline__ void set(fl4 v) { split(v, hi, lo); }
    __device__ __forceinline__ fl4 mma_b(sh4 a, fl4 c) const { return mma(a, lo, mma(a, hi, c)); }  // D += A this
};
template <>
struct SplitOp<f32_io> {
    fl4 v;
    __device__ __forceinline__ void set(fl4 x) { v = x; }
    __device__ __forceinline__ fl4 mma_b(fl4 a, fl4 c) const { return mma(a, v, c); }
};

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

// A chunk's inputs as one thread holds them between their load and their store into LDS: its share
// of b and c (rows of N), of x (rows of P) and one token's a. Which pieces a thread holds is the same
// for every chunk: Pieces fixes their token and column once.
template <typename IO>
struct ChunkRegs {
    using E = typename IO::storage;
    static constexpr int kT = SsdCfg<IO>::kT;
    static constexpr int kBC = kT * kSsdMaxState / (kSsdThreads * 8);   // 8-element pieces of b (and c)
    static constexpr int kX = kT * kSsdMaxHeadDim / (kSsdThreads * 8);  // 8-element pieces of x
    Oct<E> b[kBC], c[kBC], x[kX];
    float a;
};

template <typename IO>
struct Pieces {
    static constexpr int kBC = ChunkRegs<IO>::kBC, kX = ChunkRegs<IO>::kX;
    int bt[kBC], bn[kBC];  // token (-1: no piece) and first state of each b / c piece
    int xt[kX], xq[kX];    // token (-1: no piece) and first channel of each x piece
    __device__ __forceinline__ void init(int N, int P) {
        constexpr int kT = SsdCfg<IO>::kT;
#pragma unroll
        for (int k = 0; k < kBC; ++k) {
            const int e = (k * kSsdThreads + static_cast<int>(threadIdx.x)) * 8;
            bt[k] = e < kT * N ? e / N : -1;
            bn[k] = e < kT * N ? e - bt[k] * N : 0;
        }
#pragma unroll
        for (int k = 0; k < kX; ++k) {
            const int e = (k * kSsdThreads + static_cast<int>(threadIdx.x)) * 8;
            xt[k] = e < kT * P ? e / P : -1;
            xq[k] = e < kT * P ? e - xt[k] * P : 0;
        }
    }
};

// Load the chunk starting at token t0 (zeros past the end) into registers.
template <typename IO>
__device__ __forceinline__ void load_chunk(const SsdArgs& p, const Pieces<IO>& pc, const typename IO::storage* bbase,
                                           const typename IO::storage* cbase, const typename IO::storage* xbase,
                                           int64_t t0, ChunkRegs<IO>& r) {
    constexpr int kT = SsdCfg<IO>::kT;
    const int64_t L = p.L, bstride = p.groups * p.N, xstride = p.heads * p.P;
#pragma unroll
    for (int k = 0; k < ChunkRegs<IO>::kBC; ++k) {
        const bool in = pc.bt[k] >= 0 && t0 + pc.bt[k] < L;
        const int64_t off = in ? (t0 + pc.bt[k]) * bstride + pc.bn[k] : 0;
        r.b[k].load(bbase + off, in);
        r.c[k].load(cbase + off, in);
    }
#pragma unroll
    for (int k = 0; k < ChunkRegs<IO>::kX; ++k) {
        const bool in = pc.xt[k] >= 0 && t0 + pc.xt[k] < L;
        r.x[k].load(xbase + (in ? (t0 + pc.xt[k]) * xstride + pc.xq[k] : 0), in);
    }
    const int tl = static_cast<int>(threadIdx.x);
    r.a = tl < kT && t0 + tl < L ? p.a[(t0 + tl) * p.heads] * kLog2e : 0.0f;  // p.a already points at (b, 0, h)
}

template <typename IO>
__device__ __forceinline__ void store_chunk_lds(const Pieces<IO>& pc, const ChunkRegs<IO>& r, SsdLds<IO>& s) {
    constexpr int kT = SsdCfg<IO>::kT;
#pragma unroll
    for (int k = 0; k < ChunkRegs<IO>::kBC; ++k) {
        if (pc.bt[k] >= 0) {
            r.b[k].store(&s.b[pc.bt[k]][pc.bn[k]]);
            r.c[k].store(&s.c[pc.bt[k]][pc.bn[k]]);
        }
    }
#pragma unroll
    for (int k = 0; k < ChunkRegs<IO>::kX; ++k)
        if (pc.xt[k] >= 0) r.x[k].store(&s.x[pc.xt[k]][pc.xq[k]]);
    if (threadIdx.x < 64) {  // wave 0: inclusive prefix sum of a over the chunk (0 past the end)
        float v = threadIdx.x < kT ? r.a : 0.0f;
#pragma unroll
        for (int d = 1; d < kT; d *= 2) {
            const float o = __shfl_up(v, d, 64);
            if (static_cast<int>(threadIdx.x) >= d) v += o;
        }
        if (threadIdx.x < kT) s.acum[threadIdx.x] = v;
    }
}

// NT: 16-state blocks (N rounded up to 1, 2, 4 or 8 of them; the columns past N are zero in LDS).
template <typename IO, typename OT, int NT>
__global__ __launch_bounds__(kSsdThreads, 2) void ssd_kernel(SsdArgs p) {
    using E = typename IO::storage;
    constexpr int kT = SsdCfg<IO>::kT;
    constexpr int kTT = kT / 16;                  // 16-token blocks per chunk
    constexpr int kNT = NT;
    constexpr int kLB = kSsdMaxState + SsdCfg<IO>::kPad, kLX = kSsdMaxHeadDim + SsdCfg<IO>::kPad;
    __shared__ __align__(16) SsdLds<IO> s;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, k4 = 4 * (lane >> 4);  // operand row / column, and first of 4 k
    const int64_t H = p.heads, L = p.L;
    const int64_t bi = blockIdx.x / H, h = blockIdx.x - bi * H;
    const int64_t g = h / (H / p.groups);
    const int p0 = 16 * wave;                     // this wave's slice of the head's channels
    const bool computes = p0 < p.P;               // waves past the head's channels only stage
    // b and c columns from N up to 16 NT stay zero (the staging never writes them)
    for (int e = threadIdx.x; e < kT * (16 * NT - static_cast<int>(p.N)); e += kSsdThreads) {
        const int w = 16 * NT - static_cast<int>(p.N), t = e / w, n = static_cast<int>(p.N) + e % w;
        s.b[t][n] = E(0);
        s.c[t][n] = E(0);
    }

    fl4 z[kNT];  // the state's slice: z[nt][i] = H[p0 + r16][16 nt + k4 + i] (rows n, columns p)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) z[nt] = fl4{0.0f, 0.0f, 0.0f, 0.0f};

    using E = typename IO::storage;
    const E* bbase = static_cast<const E*>(p.b) + (bi * L * p.groups + g) * p.N;
    const E* cbase = static_cast<const E*>(p.c) + (bi * L * p.groups + g) * p.N;
    const E* xbase = static_cast<const E*>(p.x) + (bi * L * H + h) * p.P;
    SsdArgs pa = p;
    pa.a = p.a + bi * L * H + h;
    Pieces<IO> pc;
    pc.init(static_cast<int>(p.N), static_cast<int>(p.P));
    const int64_t nchunks = (L + kT - 1) / kT;
    ChunkRegs<IO> reg;
    load_chunk<IO>(pa, pc, bbase, cbase, xbase, 0, reg);
    for (int64_t ck = 0; ck < nchunks; ++ck) {
        const int64_t t0 = ck * kT;
        store_chunk_lds<IO>(pc, reg, s);
        __syncthreads();
        // the next chunk's loads are in flight while this one computes
        if (ck + 1 < nchunks) load_chunk<IO>(pa, pc, bbase, cbase, xbase, t0 + kT, reg);

        if (computes) {
            // what each 16-token block reads from the state entering the chunk, one state tile (split once)
            // at a time: yen[tt] rows t = 16 tt + k4 + i, column p = p0 + r16
            fl4 yen[kTT];
#pragma unroll
            for (int tt = 0; tt < kTT; ++tt) yen[tt] = fl4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                SplitOp<IO> zs;
                zs.set(z[nt]);
#pragma unroll
                for (int tt = 0; tt < kTT; ++tt) yen[tt] = zs.mma_b(frag_at(&s.c[16 * tt + r16][16 * nt + k4]), yen[tt]);
            }
            // ---- outputs of the chunk, one 16-token block at a time
#pragma unroll
            for (int tt = 0; tt < kTT; ++tt) {
                fl4 yin = {0.0f, 0.0f, 0.0f, 0.0f};
                const float at = s.acum[16 * tt + r16];  // row t of the transposed score tiles
#pragma unroll
                for (int st = 0; st <= tt; ++st) {
                    // scores, transposed: gt[i] = b_s . c_t with s = 16 st + k4 + i, t = 16 tt + r16
                    // (two accumulators, so that consecutive products do not wait on each other)
                    fl4 g0 = {0.0f, 0.0f, 0.0f, 0.0f}, g1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int kb = 0; kb < kNT; kb += 2) {
                        g0 = mma(frag_at(&s.b[16 * st + r16][16 * kb + k4]), frag_at(&s.c[16 * tt + r16][16 * kb + k4]), g0);
                        if (kb + 1 < kNT)
                            g1 = mma(frag_at(&s.b[16 * st + r16][16 * kb + 16 + k4]),
                                     frag_at(&s.c[16 * tt + r16][16 * kb + 16 + k4]), g1);
                    }
                    const fl4 gt = g0 + g1;
                    // masked by the decay between s and t: the A operand of the product with x (row t, k s)
                    fl4 m;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int sl = 16 * st + k4 + i, tl = 16 * tt + r16;
                        m[i] = sl <= tl ? gt[i] * exp2_hw(at - s.acum[sl]) : 0.0f;
                    }
                    yin = mma_fa(m, frag_col(&s.x[16 * st + k4][p0 + r16], kLX), yin);
                }
                // yin, yen: rows t = 16 tt + k4 + i, column p = p0 + r16
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tl = 16 * tt + k4 + i;
                    const int64_t t = t0 + tl;
                    if (t < L) {
                        const float y = fmaf(exp2_hw(s.acum[tl]), yen[tt][i], yin[i]);
                        store_out(static_cast<OT*>(p.y) + ((bi * L + t) * H + h) * p.P + p0 + r16, y);
                    }
                }
            }

            // ---- the state leaving the chunk: decayed over it, plus sum_s e^{a_{s+1}..a_end} x_s b_s^T
            const float aend = s.acum[kT - 1];
            SplitOp<IO> wx[kTT];
#pragma unroll
            for (int sb = 0; sb < kTT; ++sb) {
                fl4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int sl = 16 * sb + k4 + i;
                    v[i] = exp2_hw(aend - s.acum[sl]) * as_float<IO>(s.x[sl][p0 + r16]);
                }
                wx[sb].set(v);
            }
            const float dend = exp2_hw(aend);
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                fl4 acc = z[nt] * dend;
#pragma unroll
                for (int sb = 0; sb < kTT; ++sb) acc = wx[sb].mma_b(frag_col(&s.b[16 * sb + k4][16 * nt + r16], kLB), acc);
                z[nt] = acc;
            }
        }
        __syncthreads();  // every wave is done with the chunk's LDS before the next is stored
    }

    if (computes && p.final_state) {
        float* fs = p.final_state + ((bi * H + h) * p.P + p0 + r16) * p.N;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * nt + k4 + i < p.N) fs[16 * nt + k4 + i] = z[nt][i];
    }
}

template <typename IO, typename OT>
hipError_t launch_ssd_typed(const SsdArgs& a, hipStream_t st) {
    const uint32_t blocks = static_cast<uint32_t>(a.nb * a.heads);
    const int nt = static_cast<int>((a.N + 15) / 16);
    if (nt <= 1) hipLaunchKernelGGL((ssd_kernel<IO, OT, 1>), dim3(blocks), dim3(kSsdThreads), 0, st, a);
    else if (nt <= 2) hipLaunchKernelGGL((ssd_kernel<IO, OT, 2>), dim3(blocks), dim3(kSsdThreads), 0, st, a);
    else if (nt <= 4) hipLaunchKernelGGL((ssd_kernel<IO, OT, 4>), dim3(blocks), dim3(kSsdThreads), 0, st, a);
    else hipLaunchKernelGGL((ssd_kernel<IO, OT, 8>), dim3(blocks), dim3(kSsdThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ssd_scan(const SsdArgs& a, bool io_bf16, hipStream_t st) {
    if (!io_bf16) return launch_ssd_typed<f32_io, float>(a, st);
    return a.out_f32 ? launch_ssd_typed<bf16_io, float>(a, st) : launch_ssd_typed<bf16_io, uint16_t>(a, st);
}

}  // namespace ssm
