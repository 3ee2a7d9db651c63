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
// Mapping. Each (batch row, head)'s sequence is cut into segments of whole chunks, as many as it takes to
// give the chip about a thousand workgroups (one segment when there are enough (batch row, head) pairs).
// With several segments, a first kernel computes every segment's own contribution to the state (from a
// zero state) and its sum of a; a second turns them, in order, into the state entering each segment
// (the same recurrence, one step per segment); then one workgroup per (batch row, head, segment) walks
// its chunks in order from that state, so the state passes from chunk to chunk in registers. The waves
// of a workgroup split the head's P channels into slices of 16, each wave holding its slice of the state
// (N x 16, fp32) as matrix-core accumulators. Every product is a
// 16 x 16 tile on the matrix cores (v_mfma_f32_16x16x16_bf16 for bf16 inputs, v_mfma_f32_16x16x4_f32
// for fp32 inputs): the chunk's scores are computed transposed (b_s . c_t, a tile per pair of 16-token
// blocks with s <= t), which puts them directly in the operand layout of the next product with x.
// With bf16 inputs the products of the inputs themselves are exact; the fp32 intermediates that feed
// a second product (the masked scores, the state, the decay-weighted x) are split into a bf16 high
// part and a bf16 remainder, two products each, so the result keeps about 16 bits more than one bf16
// rounding would. The chunk's b, c and x are staged in LDS, row-major.
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {
namespace {

typedef short sh4 __attribute__((ext_vector_type(4)));
typedef short sh8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float fl4 __attribute__((ext_vector_type(4)));
typedef float fl2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename IO>
struct SsdCfg {
    // tokens per chunk: 32 keeps a workgroup's LDS (the chunk's b, c, x and score tiles) near 25 KB
    // (bf16) or 46 KB (fp32) and its registers within 3 waves per SIMD; the scores' work per token
    // grows with the chunk, the state's does not
    static constexpr int kT = 32;
    // padding per LDS row: rows stay multiples of 16 bytes (aligned 16-byte staging stores and
    // operand reads) and consecutive rows start in different banks
    static constexpr int kPad = 16 / IO::bytes;
};

// One lane's operand fragment: 4 consecutive k of a row (A operand) or of a column (B operand),
// bf16 bits or fp32 values.
__device__ __forceinline__ sh4 frag_at(const uint16_t* p) { return *reinterpret_cast<const sh4*>(p); }
__device__ __forceinline__ fl4 frag_at(const float* p) { return *reinterpret_cast<const fl4*>(p); }
// A B-operand fragment read down the columns of a 16 x 16 block in LDS (blk: its element [0][0], row
// stride `ld` elements): the lane receives rows 4 (lane / 16) + i, i = 0..3, of column lane % 16. For
// 16-bit elements this is one transposing LDS read (gfx950): within each 16 lanes, lane m fetches 4
// consecutive elements of block row m / 4 + 4 (lane / 16), columns 4 (m % 4) .. + 3, and the hardware
// hands lane j element j % 4 of the fetches of lanes j / 4 + 4 i. For fp32, four reads.
typedef __attribute__((address_space(3))) sh4 lds_sh4;
__device__ __forceinline__ sh4 frag_col_blk(const uint16_t* blk, int ld, int lane) {
    const uint16_t* q = blk + (4 * (lane >> 4) + ((lane & 15) >> 2)) * ld + 4 * (lane & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_sh4*)(q));
}
__device__ __forceinline__ fl4 frag_col_blk(const float* blk, int ld, int lane) {
    const float* q = blk + 4 * (lane >> 4) * ld + (lane & 15);
    return fl4{q[0], q[ld], q[2 * ld], q[3 * ld]};
}

// D += A B over 16 k: one bf16 instruction, or four fp32 ones (instruction j takes each lane's j-th k).
__device__ __forceinline__ fl4 mma(sh4 a, sh4 b, fl4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ fl4 mma(fl4 a, fl4 b, fl4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
}
// D += A0 B0 + A1 B1, two 16-k products given in the 16-k lane layout. With bf16 inputs this is one
// v_mfma_f32_16x16x32_bf16 (gfx950), which does twice the work of the 16-k instruction for about the
// same issue time (measured): a lane's 8 operand elements are its 4 of block 0 then its 4 of block 1,
// the same packing for A and B, so the instruction's 32 k are the two blocks' k in some order.
__device__ __forceinline__ fl4 mma2(sh4 a0, sh4 a1, sh4 b0, sh4 b1, fl4 c) {
    const sh8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    const sh8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf8, b), c, 0, 0, 0);
}
__device__ __forceinline__ fl4 mma2(fl4 a0, fl4 a1, fl4 b0, fl4 b1, fl4 c) { return mma(a1, b1, mma(a0, b0, c)); }

__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
__device__ __forceinline__ float bf16_value(uint16_t w) { return __uint_as_float(static_cast<uint32_t>(w) << 16); }

// v = hi + lo with hi, lo bf16 (round to nearest each): the error left is about 2^-16 of |v|. Values go
// in pairs through gfx950's two-value conversion to bf16; a pair's packed high parts give their fp32
// values by a shift (the low element) and a mask (the high one).
__device__ __forceinline__ void split(fl4 v, sh4& hi, sh4& lo) {
    uint32_t h[2], l[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const fl2 x = {v[2 * k], v[2 * k + 1]};
        h[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf2));
        const fl2 r = {x[0] - __uint_as_float(h[k] << 16), x[1] - __uint_as_float(h[k] & 0xffff0000u)};
        l[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf2));
    }
    hi = __builtin_bit_cast(sh4, u32x2{h[0], h[1]});
    lo = __builtin_bit_cast(sh4, u32x2{l[0], l[1]});
}

// An fp32 operand split once for several products: bf16 (hi, lo) with bf16 inputs, the value itself
// with fp32 inputs.
template <typename IO>
struct SplitOp;
template <>
struct SplitOp<bf16_io> {
    sh4 hi, lo;
    __device__ __forceinline__ void set(fl4 v) { split(v, hi, lo); }
    __device__ __forceinline__ fl4 mma_b(sh4 a, fl4 c) const { return mma(a, lo, mma(a, hi, c)); }  // D += A this
    __device__ __forceinline__ fl4 mma_a(sh4 b, fl4 c) const { return mma(lo, b, mma(hi, b, c)); }  // D += this B
    // D += A0 s0 + A1 s1 and D += s0 B0 + s1 B1 over two 16-k blocks
    static __device__ __forceinline__ fl4 mma_b2(sh4 a0, sh4 a1, const SplitOp& s0, const SplitOp& s1, fl4 c) {
        return mma2(a0, a1, s0.lo, s1.lo, mma2(a0, a1, s0.hi, s1.hi, c));
    }
    static __device__ __forceinline__ fl4 mma_a2(const SplitOp& s0, const SplitOp& s1, sh4 b0, sh4 b1, fl4 c) {
        return mma2(s0.lo, s1.lo, b0, b1, mma2(s0.hi, s1.hi, b0, b1, c));
    }
};
template <>
struct SplitOp<f32_io> {
    fl4 v;
    __device__ __forceinline__ void set(fl4 x) { v = x; }
    __device__ __forceinline__ fl4 mma_b(fl4 a, fl4 c) const { return mma(a, v, c); }
    __device__ __forceinline__ fl4 mma_a(fl4 b, fl4 c) const { return mma(v, b, c); }
    static __device__ __forceinline__ fl4 mma_b2(fl4 a0, fl4 a1, const SplitOp& s0, const SplitOp& s1, fl4 c) {
        return mma(a1, s1.v, mma(a0, s0.v, c));
    }
    static __device__ __forceinline__ fl4 mma_a2(const SplitOp& s0, const SplitOp& s1, fl4 b0, fl4 b1, fl4 c) {
        return mma(s1.v, b1, mma(s0.v, b0, c));
    }
};

template <typename IO>
struct SsdLds {
    using E = typename IO::storage;
    static constexpr int kT = SsdCfg<IO>::kT, kPad = SsdCfg<IO>::kPad;
    static constexpr int kPairs = (kT / 16) * (kT / 16 + 1) / 2;  // 16-token block pairs (s, t) with s <= t
    E b[kT][kSsdMaxState + kPad];    // [token][state]
    E c[kT][kSsdMaxState + kPad];    // [token][state]
    E x[kT][kSsdMaxHeadDim + kPad];  // [token][channel]
    float acum[kT];                  // a_{t0} + ... + a_t, times log2(e)
    float ea[2 * kT];                // 2^acum[t], then 2^(acum[kT - 1] - acum[t])
    SplitOp<IO> g[kPairs][64];       // the chunk's masked score tiles, each lane's A-operand fragment
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
    float a;   // the token's a as loaded (scaled and masked where it is used)
    bool ain;  // the token lies inside the sequence
};

template <typename IO>
struct Pieces {
    static constexpr int kBC = ChunkRegs<IO>::kBC, kX = ChunkRegs<IO>::kX;
    // per piece, its token in bits 0-7 (255: no piece) and its first column (state or channel) in bits
    // 8-15: packed, so that the positions of a thread's pieces take one register each
    uint32_t bp[kBC], xp[kX];
    __device__ __forceinline__ void init(int N, int P) {
        constexpr int kT = SsdCfg<IO>::kT;
#pragma unroll
        for (int k = 0; k < kBC; ++k) {
            const int e = (k * kSsdThreads + static_cast<int>(threadIdx.x)) * 8;
            bp[k] = e < kT * N ? static_cast<uint32_t>(e / N) | static_cast<uint32_t>(e % N) << 8 : 255u;
        }
#pragma unroll
        for (int k = 0; k < kX; ++k) {
            const int e = (k * kSsdThreads + static_cast<int>(threadIdx.x)) * 8;
            xp[k] = e < kT * P ? static_cast<uint32_t>(e / P) | static_cast<uint32_t>(e % P) << 8 : 255u;
        }
    }
    static __device__ __forceinline__ bool has(uint32_t v) { return (v & 255u) != 255u; }
    static __device__ __forceinline__ int tok(uint32_t v) { return static_cast<int>(v & 255u); }
    static __device__ __forceinline__ int col(uint32_t v) { return static_cast<int>(v >> 8); }
};

// Load the chunk starting at token t0 (zeros past the end) into registers; c only when kC.
// (Row strides in elements are below 2^24, so a piece's offset inside the chunk, token * stride +
// column, is a 32-bit product of 24-bit numbers; the chunk's own offset is uniform.)
template <typename IO, bool kC>
__device__ __forceinline__ void load_chunk(const SsdArgs& p, const Pieces<IO>& pc, const typename IO::storage* bbase,
                                           const typename IO::storage* cbase, const typename IO::storage* xbase,
                                           const float* abase, int64_t t0, ChunkRegs<IO>& r) {
    using E = typename IO::storage;
    constexpr int kT = SsdCfg<IO>::kT;
    const int bstride = static_cast<int>(p.groups * p.N), xstride = static_cast<int>(p.heads * p.P);
    const int rem = p.L - t0 < kT ? static_cast<int>(p.L - t0) : kT;  // tokens of the chunk inside the sequence
    const E* bch = bbase + t0 * bstride;
    const E* cch = cbase + t0 * bstride;
    const E* xch = xbase + t0 * xstride;
#pragma unroll
    for (int k = 0; k < ChunkRegs<IO>::kBC; ++k) {
        const uint32_t v = pc.bp[k];
        const int tok = Pieces<IO>::tok(v);
        const bool in = tok < rem;  // a missing piece has token 255
        const int off = in ? __mul24(tok, bstride) + Pieces<IO>::col(v) : 0;
        r.b[k].load(bch + off, in);
        if (kC) r.c[k].load(cch + off, in);
    }
#pragma unroll
    for (int k = 0; k < ChunkRegs<IO>::kX; ++k) {
        const uint32_t v = pc.xp[k];
        const int tok = Pieces<IO>::tok(v);
        const bool in = tok < rem;
        r.x[k].load(xch + (in ? __mul24(tok, xstride) + Pieces<IO>::col(v) : 0), in);
    }
    // a: an unconditional load of a valid element (a thread past the chunk's end reads its last token), used
    // only in store_chunk_lds. Masked or scaled here, its first use would make the compiler wait for the
    // whole chunk's loads at this point, and the next chunk's loads would no longer overlap the current
    // chunk's work.
    const int tl = static_cast<int>(threadIdx.x);
    r.a = abase[(t0 + (tl < rem ? tl : rem - 1)) * p.heads];  // abase points at (b, 0, h)
    r.ain = tl < rem;
}

template <typename IO, bool kC>
__device__ __forceinline__ void store_chunk_lds(const Pieces<IO>& pc, const ChunkRegs<IO>& r, SsdLds<IO>& s) {
    constexpr int kT = SsdCfg<IO>::kT;
#pragma unroll
    for (int k = 0; k < ChunkRegs<IO>::kBC; ++k) {
        const uint32_t v = pc.bp[k];
        if (Pieces<IO>::has(v)) {
            r.b[k].store(&s.b[Pieces<IO>::tok(v)][Pieces<IO>::col(v)]);
            if (kC) r.c[k].store(&s.c[Pieces<IO>::tok(v)][Pieces<IO>::col(v)]);
        }
    }
#pragma unroll
    for (int k = 0; k < ChunkRegs<IO>::kX; ++k)
        if (Pieces<IO>::has(pc.xp[k])) r.x[k].store(&s.x[Pieces<IO>::tok(pc.xp[k])][Pieces<IO>::col(pc.xp[k])]);
    if (threadIdx.x < 64) {  // wave 0: inclusive prefix sum of a over the chunk (0 past the end)
        float v = threadIdx.x < kT && r.ain ? r.a * kLog2e : 0.0f;
#pragma unroll
        for (int d = 1; d < kT; d *= 2) {
            const float o = __shfl_up(v, d, 64);
            if (static_cast<int>(threadIdx.x) >= d) v += o;
        }
        if (threadIdx.x < kT) s.acum[threadIdx.x] = v;
        // the decays that depend on one token: from the chunk's start to t, and from t to the chunk's end
        static_assert(2 * kT == 64, "one lane of wave 0 per decay");
        const int t = threadIdx.x & (kT - 1);
        const float vt = __shfl(v, t, 64), vend = __shfl(v, kT - 1, 64);
        s.ea[threadIdx.x] = exp2_hw(threadIdx.x < kT ? vt : vend - vt);
    }
}

// What every kernel of a launch derives from its workgroup index: the (batch row, head), the segment of
// the sequence, and where its inputs start. Workgroups are numbered (batch row, head)-major with the
// segment fastest; `nseg` is the number of segments this kernel covers per (batch row, head).
template <typename IO>
struct SsdSite {
    using E = typename IO::storage;
    int64_t bh, c0, c1;  // batch row * heads + head, and the segment's chunks [c0, c1)
    int j;               // the segment
    const E *bbase, *cbase, *xbase;
    const float* abase;  // a at (batch row, 0, head)
    int64_t ybase;       // element offset of y at (batch row, 0, head, 0)
    __device__ __forceinline__ SsdSite(const SsdArgs& p, int64_t nseg) {
        constexpr int kT = SsdCfg<IO>::kT;
        const int64_t H = p.heads, L = p.L;
        bh = blockIdx.x / nseg;
        j = static_cast<int>(blockIdx.x - bh * nseg);
        const int64_t bi = bh / H, h = bh - bi * H;
        const int64_t g = h / (H / p.groups);
        bbase = static_cast<const E*>(p.b) + (bi * L * p.groups + g) * p.N;
        cbase = static_cast<const E*>(p.c) + (bi * L * p.groups + g) * p.N;
        xbase = static_cast<const E*>(p.x) + (bi * L * H + h) * p.P;
        abase = p.a + bi * L * H + h;
        ybase = (bi * L * H + h) * p.P;
        const int64_t nchunks = ceil_div(L, kT);
        c0 = j * p.plan.seg_chunks;
        c1 = c0 + p.plan.seg_chunks < nchunks ? c0 + p.plan.seg_chunks : nchunks;
    }
    // a lane's fp32 state numbers H[prow][n ..] in the workspace's slot `slot` ([P][16 NT]: rows padded to
    // whole 16-state tiles, whose columns past N hold zeros)
    template <int NT>
    __device__ __forceinline__ float* state_slot(const SsdArgs& p, int64_t slot, int prow, int n) const {
        return p.ws_state + ((bh * (p.plan.segments - 1) + slot) * p.P + prow) * (16 * NT) + n;
    }
};

// The columns of b and c from N up to 16 NT stay zero: the staging never writes them.
template <typename IO, int NT>
__device__ __forceinline__ void zero_pad_columns(SsdLds<IO>& s, int N) {
    using E = typename IO::storage;
    constexpr int kT = SsdCfg<IO>::kT;
    const int w = 16 * NT - N;
    for (int e = threadIdx.x; e < kT * w; e += kSsdThreads) {
        const int t = e / w, n = N + e % w;
        s.b[t][n] = E(0);
        s.c[t][n] = E(0);
    }
}

// The state leaving a chunk: z <- e^{a over the chunk} z + sum_s e^{a_{s+1}..a_end} x_s b_s^T, for this
// wave's 16 channels (z[nt][i] = H[p0 + r16][16 nt + k4 + i]).
template <typename IO, int NT>
__device__ __forceinline__ void chunk_state_update(const SsdLds<IO>& s, int p0, int lane, int k4, fl4 (&z)[NT]) {
    constexpr int kT = SsdCfg<IO>::kT, kTT = kT / 16;
    constexpr int kLB = kSsdMaxState + SsdCfg<IO>::kPad, kLX = kSsdMaxHeadDim + SsdCfg<IO>::kPad;
    SplitOp<IO> wx[kTT];
#pragma unroll
    for (int sb = 0; sb < kTT; ++sb) {
        const auto xs = frag_col_blk(&s.x[16 * sb][p0], kLX, lane);  // x[16 sb + k4 + i][p0 + lane % 16]
        fl4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = s.ea[kT + 16 * sb + k4 + i] * as_float<IO>(xs[i]);
        wx[sb].set(v);
    }
    const float dend = s.ea[kT - 1];
    static_assert(kTT % 2 == 0, "the token blocks of a chunk go in pairs");
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        fl4 acc = z[nt] * dend;
#pragma unroll
        for (int sb = 0; sb < kTT; sb += 2)
            acc = SplitOp<IO>::mma_b2(frag_col_blk(&s.b[16 * sb][16 * nt], kLB, lane),
                                      frag_col_blk(&s.b[16 * sb + 16][16 * nt], kLB, lane), wx[sb], wx[sb + 1], acc);
        z[nt] = acc;
    }
}

// The chunk's scores, transposed and masked by the decay, into LDS: for every pair of 16-token blocks
// s <= t, tile[s-row i][t] = (b_s . c_t) e^{a_{s+1}+...+a_t} (0 above the diagonal), as each lane's
// A-operand fragment of the product with x (row t = r16, k = s = k4 .. k4 + 3). The scores do not depend
// on the channel, so the workgroup's waves share the tiles out and compute each once.
template <typename IO, int NT>
__device__ __forceinline__ void chunk_scores(SsdLds<IO>& s, int wave, int lane, int r16, int k4) {
    constexpr int kPairs = SsdLds<IO>::kPairs, kWaves = kSsdThreads / 64;
    for (int pi = wave; pi < kPairs; pi += kWaves) {
        int tt = 0;  // pi = tt (tt + 1) / 2 + st
        while ((tt + 1) * (tt + 2) / 2 <= pi) ++tt;
        const int st = pi - tt * (tt + 1) / 2;
        // (pairs of 16-state blocks per product; two accumulators, so that consecutive products do not
        // wait on each other)
        fl4 g0 = {0.0f, 0.0f, 0.0f, 0.0f}, g1 = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (NT == 1) {
            g0 = mma(frag_at(&s.b[16 * st + r16][k4]), frag_at(&s.c[16 * tt + r16][k4]), g0);
        } else {
#pragma unroll
            for (int kb = 0; kb < NT; kb += 2) {
                const auto bf0 = frag_at(&s.b[16 * st + r16][16 * kb + k4]), bf1 = frag_at(&s.b[16 * st + r16][16 * kb + 16 + k4]);
                const auto cf0 = frag_at(&s.c[16 * tt + r16][16 * kb + k4]), cf1 = frag_at(&s.c[16 * tt + r16][16 * kb + 16 + k4]);
                if ((kb / 2) % 2 == 0) g0 = mma2(bf0, bf1, cf0, cf1, g0);
                else g1 = mma2(bf0, bf1, cf0, cf1, g1);
            }
        }
        const fl4 gt = g0 + g1;  // gt[i] = b_s . c_t, s = 16 st + k4 + i, t = 16 tt + r16
        const float at = s.acum[16 * tt + r16];
        fl4 m;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int sl = 16 * st + k4 + i, tl = 16 * tt + r16;
            m[i] = sl <= tl ? gt[i] * exp2_hw(at - s.acum[sl]) : 0.0f;
        }
        SplitOp<IO> ms;
        ms.set(m);
        s.g[pi][lane] = ms;
    }
}

// What each 16-token block reads from the state entering the chunk, one state tile (split once) at a
// time: yen[tt][i] = sum_n c[16 tt + k4 + i][n] H[p0 + r16][n].
template <typename IO, int NT>
__device__ __forceinline__ void chunk_entering(const SsdLds<IO>& s, int r16, int k4, const fl4 (&z)[NT],
                                               fl4 (&yen)[SsdCfg<IO>::kT / 16]) {
    constexpr int kTT = SsdCfg<IO>::kT / 16;
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) yen[tt] = fl4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (NT == 1) {
        SplitOp<IO> zs;
        zs.set(z[0]);
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt) yen[tt] = zs.mma_b(frag_at(&s.c[16 * tt + r16][k4]), yen[tt]);
    } else {
#pragma unroll
        for (int nt = 0; nt < NT; nt += 2) {
            SplitOp<IO> z0, z1;
            z0.set(z[nt]);
            z1.set(z[nt + 1]);
#pragma unroll
            for (int tt = 0; tt < kTT; ++tt)
                yen[tt] = SplitOp<IO>::mma_b2(frag_at(&s.c[16 * tt + r16][16 * nt + k4]),
                                              frag_at(&s.c[16 * tt + r16][16 * nt + 16 + k4]), z0, z1, yen[tt]);
        }
    }
}

// The outputs of one chunk of kT tokens starting at t0: the masked scores (LDS) applied to x, plus the
// entering state's part scaled by e^{a_{t0}+...+a_t}.
template <typename IO, typename OT>
__device__ __forceinline__ void chunk_outputs(const SsdArgs& p, const SsdLds<IO>& s, OT* y, int64_t t0, int p0, int lane,
                                              int r16, int k4, const fl4 (&yen)[SsdCfg<IO>::kT / 16]) {
    constexpr int kT = SsdCfg<IO>::kT, kTT = kT / 16;
    constexpr int kLX = kSsdMaxHeadDim + SsdCfg<IO>::kPad;
    // y points at (batch row, 0, head, 0); this lane writes rows t0 + k4 + 16 tt + i of column p0 + r16
    const int ystride = static_cast<int>(p.heads * p.P);
    OT* yl = y + t0 * ystride + __mul24(k4, ystride) + p0 + r16;
    const int rem = p.L - t0 - k4 < kT ? static_cast<int>(p.L - t0 - k4) : kT;  // rows of this lane in the sequence
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
        fl4 yin = {0.0f, 0.0f, 0.0f, 0.0f};
        const int pb = tt * (tt + 1) / 2;  // the tiles (tt, 0 .. tt), in pairs of blocks s
#pragma unroll
        for (int st = 0; st + 1 <= tt; st += 2)
            yin = SplitOp<IO>::mma_a2(s.g[pb + st][lane], s.g[pb + st + 1][lane], frag_col_blk(&s.x[16 * st][p0], kLX, lane),
                                      frag_col_blk(&s.x[16 * st + 16][p0], kLX, lane), yin);
        if (tt % 2 == 0) yin = s.g[pb + tt][lane].mma_a(frag_col_blk(&s.x[16 * tt][p0], kLX, lane), yin);
        // yin, yen: rows t = 16 tt + k4 + i, column p = p0 + r16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tl = 16 * tt + k4 + i;
            if (16 * tt + i < rem) store_out(yl + (16 * tt + i) * ystride, fmaf(s.ea[tl], yen[tt][i], yin[i]));
        }
    }
}

// NT: 16-state blocks (N rounded up to 1, 2, 4 or 8 of them; the columns past N are zero in LDS).
// One workgroup per (batch row, head, segment): the segment's outputs from the state entering it (zero
// for the first segment, else the workspace's carry), walking its chunks in order; the last segment
// writes the final state.
template <typename IO, typename OT, int NT>
__global__ __launch_bounds__(kSsdThreads, 3) void ssd_kernel(SsdArgs p) {
    constexpr int kT = SsdCfg<IO>::kT;
    __shared__ __align__(16) SsdLds<IO> s;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, k4 = 4 * (lane >> 4);  // operand row / column, and first of 4 k
    const int p0 = 16 * wave;                          // this wave's slice of the head's channels
    const bool computes = p0 < p.P;                    // waves past the head's channels only stage
    const SsdSite<IO> site(p, p.plan.segments);
    zero_pad_columns<IO, NT>(s, static_cast<int>(p.N));

    fl4 z[NT];  // the state's slice: z[nt][i] = H[p0 + r16][16 nt + k4 + i]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        z[nt] = fl4{0.0f, 0.0f, 0.0f, 0.0f};
        if (site.j > 0 && computes)
            z[nt] = *reinterpret_cast<const fl4*>(site.template state_slot<NT>(p, site.j - 1, p0 + r16, 16 * nt + k4));
    }

    Pieces<IO> pc;
    pc.init(static_cast<int>(p.N), static_cast<int>(p.P));
    ChunkRegs<IO> reg;
    load_chunk<IO, true>(p, pc, site.bbase, site.cbase, site.xbase, site.abase, site.c0 * kT, reg);
    const int nck = static_cast<int>(site.c1 - site.c0);
    int64_t t0 = site.c0 * kT;
    for (int ck = 0; ck < nck; ++ck, t0 += kT) {
        store_chunk_lds<IO, true>(pc, reg, s);
        __syncthreads();
        // the next chunk's loads are in flight while this one computes
        if (ck + 1 < nck) load_chunk<IO, true>(p, pc, site.bbase, site.cbase, site.xbase, site.abase, t0 + kT, reg);
        chunk_scores<IO, NT>(s, wave, lane, r16, k4);
        fl4 yen[kT / 16];
        if (computes) chunk_entering<IO, NT>(s, r16, k4, z, yen);
        __syncthreads();  // the score tiles are in LDS
        if (computes) {
            chunk_outputs<IO, OT>(p, s, static_cast<OT*>(p.y) + site.ybase, t0, p0, lane, r16, k4, yen);
            chunk_state_update<IO, NT>(s, p0, lane, k4, z);
        }
        __syncthreads();  // every wave is done with the chunk's LDS before the next is stored
    }

    if (computes && p.final_state && site.j == p.plan.segments - 1) {
        float* fs = p.final_state + (site.bh * p.P + p0 + r16) * p.N;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            if (16 * nt < p.N) *reinterpret_cast<fl4*>(fs + 16 * nt + k4) = z[nt];
    }
}

// One workgroup per (batch row, head, segment) but the last: the segment's own contribution to the
// state (from a zero state) and its sum of a, into the workspace.
template <typename IO, int NT>
__global__ __launch_bounds__(kSsdThreads, 3) void ssd_segment_state_kernel(SsdArgs p) {
    constexpr int kT = SsdCfg<IO>::kT;
    __shared__ __align__(16) SsdLds<IO> s;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, k4 = 4 * (lane >> 4);
    const int p0 = 16 * wave;
    const bool computes = p0 < p.P;
    const SsdSite<IO> site(p, p.plan.segments - 1);
    zero_pad_columns<IO, NT>(s, static_cast<int>(p.N));

    fl4 z[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) z[nt] = fl4{0.0f, 0.0f, 0.0f, 0.0f};
    float asum = 0.0f;  // the segment's sum of a (times log2 e), the same in every lane

    Pieces<IO> pc;
    pc.init(static_cast<int>(p.N), static_cast<int>(p.P));
    ChunkRegs<IO> reg;
    load_chunk<IO, false>(p, pc, site.bbase, site.cbase, site.xbase, site.abase, site.c0 * kT, reg);
    const int nck = static_cast<int>(site.c1 - site.c0);
    int64_t t0 = site.c0 * kT;
    for (int ck = 0; ck < nck; ++ck, t0 += kT) {
        store_chunk_lds<IO, false>(pc, reg, s);
        __syncthreads();
        if (ck + 1 < nck) load_chunk<IO, false>(p, pc, site.bbase, site.cbase, site.xbase, site.abase, t0 + kT, reg);
        asum += s.acum[kT - 1];
        if (computes) chunk_state_update<IO, NT>(s, p0, lane, k4, z);
        __syncthreads();
    }

    if (computes) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            *reinterpret_cast<fl4*>(site.template state_slot<NT>(p, site.j, p0 + r16, 16 * nt + k4)) = z[nt];
    }
    if (threadIdx.x == 0) p.ws_decay[site.bh * p.plan.segments + site.j] = asum;
}

// One thread per state number of every (batch row, head): turns the segments' own contributions into
// the states entering the segments after them, H_in(k+1) = e^{a over segment k} H_in(k) + S_k with
// H_in(0) = 0, in place (slot k receives the state entering segment k + 1).
__global__ __launch_bounds__(256) void ssd_carry_kernel(float* ws_state, const float* ws_decay, int64_t nbh, int64_t pn,
                                                        int64_t nseg) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= nbh * pn) return;
    const int64_t bh = i / pn, e = i - bh * pn;
    float* st = ws_state + bh * (nseg - 1) * pn + e;
    const float* dec = ws_decay + bh * nseg;
    float sk[kSsdMaxSegments - 1];  // every slot's load is issued before the first fold
#pragma unroll
    for (int k = 0; k < kSsdMaxSegments - 1; ++k)
        if (k < nseg - 1) sk[k] = st[k * pn];
    float hin = 0.0f;
#pragma unroll
    for (int k = 0; k < kSsdMaxSegments - 1; ++k) {
        if (k < nseg - 1) {
            hin = fmaf(exp2_hw(dec[k]), hin, sk[k]);
            st[k * pn] = hin;
        }
    }
}

template <typename IO, typename OT, int NT>
hipError_t launch_ssd_nt(const SsdArgs& a, hipStream_t st) {
    const int64_t bh = a.nb * a.heads, nseg = a.plan.segments;
    if (nseg > 1) {
        hipLaunchKernelGGL((ssd_segment_state_kernel<IO, NT>), dim3(static_cast<uint32_t>(bh * (nseg - 1))),
                           dim3(kSsdThreads), 0, st, a);
        const int64_t pn = a.P * 16 * NT, n = bh * pn;
        hipLaunchKernelGGL(ssd_carry_kernel, dim3(static_cast<uint32_t>(ceil_div(n, 256))), dim3(256), 0, st,
                           a.ws_state, static_cast<const float*>(a.ws_decay), bh, pn, nseg);
    }
    hipLaunchKernelGGL((ssd_kernel<IO, OT, NT>), dim3(static_cast<uint32_t>(bh * nseg)), dim3(kSsdThreads), 0, st, a);
    return hipGetLastError();
}

template <typename IO, typename OT>
hipError_t launch_ssd_typed(const SsdArgs& a, hipStream_t st) {
    switch (ssd_state_cols(a.N)) {
        case 16: return launch_ssd_nt<IO, OT, 1>(a, st);
        case 32: return launch_ssd_nt<IO, OT, 2>(a, st);
        case 64: return launch_ssd_nt<IO, OT, 4>(a, st);
        default: return launch_ssd_nt<IO, OT, 8>(a, st);
    }
}

// Workgroups a launch aims for: enough to give every CU a few, so that a shape with few (batch row, head)
// pairs still fills the chip; more only adds state traffic.
constexpr int64_t kSsdTargetBlocks = 1024;

}  // namespace

int64_t ssd_state_cols(int64_t N) {
    const int64_t nt = ceil_div(N, 16);
    return 16 * (nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : 8);
}

SsdPlan ssd_plan(int64_t nb, int64_t L, int64_t heads, bool io_bf16, bool split) {
    const int64_t kT = io_bf16 ? SsdCfg<bf16_io>::kT : SsdCfg<f32_io>::kT;
    const int64_t nchunks = ceil_div(L, kT), bh = nb * heads;
    int64_t seg = split ? ceil_div(kSsdTargetBlocks, bh) : 1;
    if (seg > kSsdMaxSegments) seg = kSsdMaxSegments;
    if (seg > nchunks) seg = nchunks;
    if (seg <= 1) return SsdPlan{1, nchunks};
    const int64_t per = ceil_div(nchunks, seg);
    return SsdPlan{ceil_div(nchunks, per), per};
}

size_t ssd_workspace_bytes(const SsdPlan& plan, int64_t nb, int64_t heads, int64_t P, int64_t N) {
    if (plan.segments <= 1) return 0;
    const size_t bh = static_cast<size_t>(nb * heads);
    const size_t dec = (bh * plan.segments * sizeof(float) + 255) / 256 * 256;
    return dec + bh * (plan.segments - 1) * P * ssd_state_cols(N) * sizeof(float);
}

hipError_t launch_ssd_scan(SsdArgs a, bool io_bf16, void* workspace, hipStream_t st) {
    if (a.plan.segments > 1) {
        const size_t bh = static_cast<size_t>(a.nb * a.heads);
        a.ws_decay = static_cast<float*>(workspace);
        a.ws_state = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                              (bh * a.plan.segments * sizeof(float) + 255) / 256 * 256);
    } else {
        a.ws_decay = a.ws_state = nullptr;
    }
    if (!io_bf16) return launch_ssd_typed<f32_io, float>(a, st);
    return a.out_f32 ? launch_ssd_typed<bf16_io, float>(a, st) : launch_ssd_typed<bf16_io, uint16_t>(a, st);
}

}  // namespace ssm
