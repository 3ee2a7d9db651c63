// scan_bwd.hip - backward of the selective scan (gfx950, Euler input gain).
//
// Given dout = dL/dout, the gradients of every input of the forward scan. With h_t = a_t h_{t-1}
// + Delta_t B_t u_t (a_t = exp(Delta_t A)), y_t = sum_n C_t h_t + D u_t, out_t = y_t SiLU(z_t) and
// dy_t = dout_t SiLU(z_t), the adjoint of h_t runs backwards in time,
//   lambda_t = C_t dy_t + a_{t+1} lambda_{t+1},
// and every term of the forward pass hands its partial derivative to the inputs (the same algebra
// as the fp64 oracle; "Beyond attention with Mamba, state space models and hybrids", section 6: the
// fused kernel recomputes the states for the backward pass instead of storing them).
//
// The pass is a chain of kernels on one stream, none of which waits on another workgroup:
//   1. the forward kernel in checkpoint mode writes the state entering each 16-token block; then,
//      per block, the adjoint from zero at the block's end: its value after the block's first decay
//      (mu = a_first lambda_first) and the block's decay 2^(a2 sum Delta) form the block's affine
//      aggregate, as in the forward pass but in reverse;
//      the 4 blocks of each 64-token segment are composed into the segment's aggregate;
//   2. segment_carry_kernel: per (channel, state), the carries into every segment from the right,
//      composing those aggregates from the end of the sequence (the carry into a block is folded
//      from its segment's by the gradient kernel, over the segment's blocks to its right);
//   3. grad_kernel: per block, the states recomputed from the checkpoint (2 states at a time, the
//      16 tokens kept in registers), then the adjoint backwards through the block with every
//      gradient term; the sums over channels (dB, dC) are folded across the wave in registers into
//      per-group partials, the sums over tokens (dA, dD, dbias) go into per-workgroup partials;
//   4. reduce_bc_kernel, reduce_channel_kernel: the partials summed into the outputs.
// Layout: lanes = 64 channels of one batch row, a wave = one 16-token block, as in the forward.
#include "scan_common.hpp"
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {
namespace {

using namespace scan;

constexpr int kWavesB = 4;  // blocks per workgroup
constexpr int kThreadsB = kWavesB * 64;
constexpr int kGS = 2;      // states per pass of the gradient kernel (the block's states of them kept)
constexpr int kNV = 2 * kGS;  // dB and dC values per token and pass, summed over the channels
static_assert(kNV == 4 && kTok == 16, "the channel sums fold 8 tokens x 4 values per lane, twice per block");

// Sums over the wave's 64 channels of 8 tokens x 4 values per lane (value k = 4 token + kind), by halving:
// each stage pairs values whose index differs in one bit with lanes that differ in one bit, and every lane
// keeps one value of each pair summed with its partner lane's copy (lanes with the lane bit clear keep the
// first). Lane distances 32 and 16 use gfx950's permlane swaps (the 32-lane swap of (x, y) hands lanes
// < 32 the x of lane + 32 and lanes >= 32 the y of lane - 32; the 16-lane swap does the same between
// 16-lane rows), distances 8, 4 and 2 DPP row shifts and a select, distance 1 a DPP quad permutation.
// Lane l returns the total of token 4 b5 + 2 b4 + b3, kind 2 b2 + b1 (bK = bit K of l); lanes l and
// l ^ 1 hold the same total.
__device__ __forceinline__ float swap_fold32(float x, float y) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_fold16(float x, float y) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// distance D in {2, 4, 8} within 16-lane rows: lanes with bit D clear get x + x[lane + D], the others
// y + y[lane - D] (row_shl:D, row_shr:D); `sel` is all ones in the lanes with bit D set
template <int D>
__device__ __forceinline__ float row_fold(float x, float y, int sel) {
    const float lo = x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x100 + D, 0xf, 0xf, true));
    const float hi = y + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0x110 + D, 0xf, 0xf, true));
    return __int_as_float((sel & __float_as_int(hi)) | (~sel & __float_as_int(lo)));
}
__device__ __forceinline__ float wave_fold32(const float (&v)[8][4], int sel8, int sel4, int sel2) {
    float a[4][4], b[2][4], c[4], d[2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int k = 0; k < 4; ++k) a[t][k] = swap_fold32(v[t][k], v[t + 4][k]);  // token bit 2
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int k = 0; k < 4; ++k) b[t][k] = swap_fold16(a[t][k], a[t + 2][k]);  // token bit 1
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = row_fold<8>(b[0][k], b[1][k], sel8);     // token bit 0
#pragma unroll
    for (int k = 0; k < 2; ++k) d[k] = row_fold<4>(c[k], c[k + 2], sel4);       // kind bit 1
    const float e = row_fold<2>(d[0], d[1], sel2);                              // kind bit 0
    return e + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(e), 0xb1, 0xf, 0xf, true));  // lane ^ 1
}


// Per-wave index set: batch row, channel, block.
struct WaveIdx {
    int wave, lane;
    int64_t b, d0, d, dc, blk, t0, row;
    bool active;
};

__device__ __forceinline__ WaveIdx wave_index(const BwdArgs& q) {
    WaveIdx w;
    w.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    w.lane = threadIdx.x & 63;
    const int64_t seg = blockIdx.x / q.nbg;  // segment of kWavesB blocks
    const int64_t bg = blockIdx.x - seg * q.nbg;
    w.b = bg / q.groups;
    w.d0 = (bg - w.b * q.groups) * 64;
    w.d = w.d0 + w.lane;
    w.active = w.d < q.a.nd;
    w.dc = w.active ? w.d : q.a.nd - 1;
    w.blk = seg * kWavesB + w.wave;
    w.t0 = w.blk * kTok;  // may lie past the end in the last segment: such a block contributes nothing
    w.row = w.b * q.a.nd + w.dc;  // (batch row, channel) index
    return w;
}

// Step Delta (0 past the end) and, with softplus, its derivative sigmoid(r) for one wave's tokens, from
// the raw delta row (loaded earlier with the block's other inputs).
template <typename IO, bool SP>
__device__ __forceinline__ void block_steps(const TokRow<IO>& dr, float bias, int64_t t0, int64_t L, float (&dt)[kTok],
                                            float (&dsp)[kTok]) {
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
        const float r = dr.get(j) + bias;
        const bool in = t0 + j < L;
        dt[j] = in ? (SP ? softplus_f32(r) : r) : 0.0f;
        dsp[j] = SP ? __builtin_amdgcn_rcpf(1.0f + exp2_hw(-r * kLog2e)) : 1.0f;
    }
}

// dy = dout * SiLU(z) (dout alone without a gate), zero past the end; with the gate also
// gz = dout * SiLU'(z), SiLU'(z) = sigmoid(z) (1 + z (1 - sigmoid(z))), for dz = gz * y.
template <typename IO, bool GZ>
__device__ __forceinline__ void block_dy(const TokRow<IO>& dor, const TokRow<IO>& zr, float (&dy)[kTok],
                                         float (&gz)[kTok]) {
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
        dy[j] = dor.get(j);
        if constexpr (GZ) {
            const float zz = zr.get(j);
            const float sg = __builtin_amdgcn_rcpf(1.0f + exp2_hw(-zz * kLog2e));
            gz[j] = dy[j] * (sg * fmaf(zz, 1.0f - sg, 1.0f));
            dy[j] *= zz * sg;
        }
    }
}

// A[d, n] for a state n that may lie past N: an unconditional load of a valid element (no branch
// around the load, so it can be issued together with others), zero past N.
__device__ __forceinline__ float a_elem(const float* __restrict__ A, int64_t d, int n, int N) {
    const float v = A[d * N + (n < N ? n : N - 1)];
    return n < N ? v : 0.0f;
}

// ---- 2. carries into each 64-token segment from the right: one lane per (batch row x channel group,
// state, channel), walking the segments' reverse aggregates from the end of the sequence
__global__ __launch_bounds__(256) void segment_carry_kernel(BwdArgs q) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= q.nbg * kMaxState * 64) return;
    const int lane = static_cast<int>(gid % 64);
    const int n = static_cast<int>((gid / 64) % kMaxState);
    const int64_t bg = gid / (64 * kMaxState);
    const int64_t g = bg % q.groups;
    const int64_t d = g * 64 + lane < q.a.nd ? g * 64 + lane : q.a.nd - 1;
    const int N = q.a.N;
    const float a2 = n < N ? q.a.A[d * N + n] * kLog2e : 0.0f;
    const float* agg = q.segagg + bg * q.nseg * (kMaxState + 1) * 64 + lane;
    float* car = q.segcarry + bg * q.nseg * kMaxState * 64 + n * 64 + lane;
    float e = 0.0f;  // nothing enters the last segment from the right
    int64_t k = q.nseg - 1;
    constexpr int kU = 8;  // segments whose loads are issued together (the chain through e stays serial)
    for (; k >= kU - 1; k -= kU) {
        float mv[kU], sv[kU];
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            mv[i] = agg[((k - i) * (kMaxState + 1) + n) * 64];
            sv[i] = agg[((k - i) * (kMaxState + 1) + kMaxState) * 64];
        }
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            car[(k - i) * kMaxState * 64] = e;
            e = fmaf(exp2_hw(a2 * sv[i]), e, mv[i]);
        }
    }
    for (; k >= 0; --k) {
        car[k * kMaxState * 64] = e;
        e = fmaf(exp2_hw(a2 * agg[(k * (kMaxState + 1) + kMaxState) * 64]), e, agg[(k * (kMaxState + 1) + n) * 64]);
    }
}

// ---- 3. gradients of one block
template <typename IO, int NFIX, bool VEC, bool SP, bool GZ>
__global__ __launch_bounds__(kThreadsB, 2) void grad_kernel(BwdArgs q) {
    using T = typename IO::storage;
    __shared__ __align__(16) float s_rows[kWavesB][2][kTok][kMaxState];
    __shared__ float s_acc[kWavesB][kMaxState + 2][64];  // per wave: dA (16 states), dD, dbias
    __shared__ float s_fin[kWavesB][2][kTok][64];       // per wave and token: sigmoid(r) and gz, for the end
    const WaveIdx w = wave_index(q);
    const int N = NFIX == kMaxState ? kMaxState : q.a.N;
    const int64_t L = q.a.L;
    // Every input load of the block is issued before any of them is used (the compiler waits for a loaded
    // value at its first use, in issue order), so the block pays one memory round trip before its passes
    // instead of one per input: the B and C rows as raw words, bias and D, delta, dout, z and u in the io
    // format, the adjoint carried in from the right, and A.
    const bool rows_fast = NFIX == kMaxState && w.t0 + kTok <= L;
    RowWords<IO> rbw, rcw;
    if (rows_fast) {
        fetch_rows<IO>(static_cast<const T*>(q.a.B) + w.b * L * N, w.t0, w.lane, rbw);
        fetch_rows<IO>(static_cast<const T*>(q.a.C) + w.b * L * N, w.t0, w.lane, rcw);
    }
    const float bias = q.a.delta_bias ? q.a.delta_bias[w.dc] : 0.0f;
    const float skip = q.a.D ? q.a.D[w.dc] : 0.0f;
    TokRow<IO> dr, dor, zr, ur;
    load_tokrow<VEC>(static_cast<const T*>(q.a.delta) + w.row * L, w.t0, L, dr);
    load_tokrow<VEC>(static_cast<const T*>(q.dout) + w.row * L, w.t0, L, dor);
    if constexpr (GZ) load_tokrow<VEC>(static_cast<const T*>(q.a.z) + w.row * L, w.t0, L, zr);
    load_tokrow<VEC>(static_cast<const T*>(q.a.u) + w.row * L, w.t0, L, ur);
    // the adjoint carried into this block from the right: the segment's carry taken over the blocks
    // after this one in the segment (their reverse aggregate from zero and their step sum, composed by
    // the checkpoint pass)
    const int64_t sb = (w.b * q.groups + w.d0 / 64) * q.nseg + w.blk / kWavesB;
    float cv[kMaxState], rv[kMaxState], av[kMaxState];  // av: A[d, n]
    float ssuf;
    {
        const float* ec = q.segcarry + sb * kMaxState * 64 + w.lane;
        const float* sf = q.lam + (sb * kWavesB + w.wave) * kMaxState * 64 + w.lane;
        ssuf = q.sdt[(sb * kWavesB + w.wave) * 64 + w.lane];
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) {
            cv[n] = ec[n * 64];
            rv[n] = sf[n * 64];
        }
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) av[n] = a_elem(q.a.A, w.dc, n, N);
    }

    if (rows_fast) {
        put_rows<IO>(rbw, w.lane, s_rows[w.wave][0]);
        put_rows<IO>(rcw, w.lane, s_rows[w.wave][1]);
    } else {
        stage_rows<IO, 0>(static_cast<const T*>(q.a.B) + w.b * L * N, w.t0, L, N, w.lane, s_rows[w.wave][0]);
        stage_rows<IO, 0>(static_cast<const T*>(q.a.C) + w.b * L * N, w.t0, L, N, w.lane, s_rows[w.wave][1]);
    }
    float dt[kTok], dy[kTok];
    {
        // the softplus derivative and the gate's factor are not held across the passes but parked in
        // LDS for the final per-token terms
        float dsp[kTok], gz[kTok];
        block_steps<IO, SP>(dr, bias, w.t0, L, dt, dsp);
        block_dy<IO, GZ>(dor, zr, dy, gz);
#pragma unroll
        for (int j = 0; j < kTok; ++j) {
            if constexpr (SP) s_fin[w.wave][0][j][w.lane] = dsp[j];
            if constexpr (GZ) s_fin[w.wave][1][j][w.lane] = gz[j];
        }
    }
    if (!w.active) {  // a lane past the last channel (it reads that channel) adds nothing to dB and dC
#pragma unroll
        for (int j = 0; j < kTok; ++j) dt[j] = dy[j] = 0.0f;
    }
    float dx[kTok];  // Delta u, the input's weight in every state and in dB
#pragma unroll
    for (int j = 0; j < kTok; ++j) dx[j] = dt[j] * ur.get(j);

    // per token, summed over the states: q A (for dDelta), l B (for du and dDelta) and the readout C h
    // (for dz)
    float ddt[kTok], lbs[kTok], ypre[kTok];
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
        ddt[j] = 0.0f;
        lbs[j] = 0.0f;
        ypre[j] = 0.0f;
    }
    // a block past the end reads the last block's checkpoint (valid memory); with zero steps, dy and u
    // it adds exactly nothing
    const int64_t blk_r = w.blk < q.nblk ? w.blk : q.nblk - 1;
    const float* hin = q.hblk + (w.row * q.nblk + blk_r) * kMaxState;
    // the entering adjoint per state, kept in s_acc's rows until the pass that needs it (a pass overwrites
    // only rows already read)
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) s_acc[w.wave][n][w.lane] = fmaf(exp2_hw(av[n] * kLog2e * ssuf), cv[n], rv[n]);
    // the channel sums of every 8 tokens: lane -> (token tk, kind: dB or dC, state of the pair); even lanes
    // store, into the partial of this channel group at the pass's first state
    const int sel8 = w.lane & 8 ? -1 : 0, sel4 = w.lane & 4 ? -1 : 0, sel2 = w.lane & 2 ? -1 : 0;
    const int tk = 4 * ((w.lane >> 5) & 1) + 2 * ((w.lane >> 4) & 1) + ((w.lane >> 3) & 1);
    float* const part_l = ((w.lane & 4) ? q.dCp : q.dBp) + ((w.d0 / 64 * q.a.nb + w.b) * L + w.t0 + tk) * kMaxState +
                          ((w.lane >> 1) & 1);
    const bool stores = !(w.lane & 1);

    // the checkpoint and the entering adjoint of the next kGS states are loaded one pass ahead
    float h0n[kGS], mun[kGS], ann[kGS];
#pragma unroll
    for (int i = 0; i < kGS; ++i) {
        h0n[i] = hin[i];
        mun[i] = s_acc[w.wave][i][w.lane];
        ann[i] = av[i];
    }
#pragma unroll 1
    for (int g = 0; g < kMaxState / kGS; ++g) {  // kGS states at a time
        float a2[kGS], an[kGS], h0[kGS], mu[kGS], dAacc[kGS];
#pragma unroll
        for (int i = 0; i < kGS; ++i) {
            an[i] = ann[i];
            a2[i] = an[i] * kLog2e;
            h0[i] = h0n[i];
            mu[i] = mun[i];
            dAacc[i] = 0.0f;
        }
        if (g + 1 < kMaxState / kGS) {
#pragma unroll
            for (int i = 0; i < kGS; ++i) {
                h0n[i] = hin[kGS * (g + 1) + i];
                mun[i] = s_acc[w.wave][kGS * (g + 1) + i][w.lane];
                ann[i] = a_elem(q.a.A, w.dc, kGS * (g + 1) + i, N);
            }
        }
        // forward: the states of the block's 16 tokens for these kGS states. The decays first (they do
        // not depend on the states, and back-to-back exponentials issue faster), then the recurrence, each
        // token's B values read from LDS one token ahead.
        float hs[kTok][kGS], as[kTok][kGS];  // the states and their decays, for the backward sweep
#pragma unroll
        for (int j = 0; j < kTok; ++j)
#pragma unroll
            for (int i = 0; i < kGS; ++i) as[j][i] = exp2_hw(dt[j] * a2[i]);
        __builtin_amdgcn_sched_barrier(0);
        float2 bnext = *reinterpret_cast<const float2*>(&s_rows[w.wave][0][0][kGS * g]);
#pragma unroll
        for (int j = 0; j < kTok; ++j) {
            const float2 bq = bnext;
            if (j + 1 < kTok) bnext = *reinterpret_cast<const float2*>(&s_rows[w.wave][0][j + 1][kGS * g]);
            const float bv[kGS] = {bq.x, bq.y};
#pragma unroll
            for (int i = 0; i < kGS; ++i) hs[j][i] = pin(fmaf(as[j][i], j > 0 ? hs[j - 1][i] : h0[i], bv[i] * dx[j]));
        }
        __builtin_amdgcn_sched_barrier(0);
        // backward through the block (B and C read one token ahead)
        float fold[8][kNV];  // dB, dC terms of the last 8 tokens, per lane
        float2 bprev = *reinterpret_cast<const float2*>(&s_rows[w.wave][0][kTok - 1][kGS * g]);
        float2 cprev = *reinterpret_cast<const float2*>(&s_rows[w.wave][1][kTok - 1][kGS * g]);
#pragma unroll
        for (int j = kTok - 1; j >= 0; --j) {
            const float dtj = dt[j], dyj = dy[j], dxj = dx[j];
            const float2 bq = bprev, cq = cprev;
            if (j > 0) {
                bprev = *reinterpret_cast<const float2*>(&s_rows[w.wave][0][j - 1][kGS * g]);
                cprev = *reinterpret_cast<const float2*>(&s_rows[w.wave][1][j - 1][kGS * g]);
            }
            const float bv[kGS] = {bq.x, bq.y}, cv[kGS] = {cq.x, cq.y};
            // the dB and dC terms of tokens 8-15 summed over the wave's 64 channels, in registers, while
            // token 7 computes (the same scheduling region); those of tokens 0-7 after token 0
            if (j == 7) {
                const float sum = wave_fold32(fold, sel8, sel4, sel2);
                if (stores && w.t0 + 8 + tk < L) part_l[8 * kMaxState + kGS * g] = sum;
            }
            // with l = lambda_t and q = l a h_{t-1}: dA += q Delta, dDelta += q A + u sum_n l B,
            // du += Delta sum_n l B, dB[t, n] = sum_d l Delta u, dC[t, n] = sum_d dy h
            float yp = 0.0f;
            float(&red)[kNV] = fold[j % 8];
#pragma unroll
            for (int i = 0; i < kGS; ++i) {
                const float l = fmaf(cv[i], dyj, mu[i]);
                const float a = as[j][i];
                const float hp = j > 0 ? hs[j - 1][i] : h0[i];
                const float qv = l * (hp * a);
                dAacc[i] = fmaf(qv, dtj, dAacc[i]);
                ddt[j] = fmaf(qv, an[i], ddt[j]);
                lbs[j] = fmaf(l, bv[i], lbs[j]);
                if constexpr (GZ) yp = fmaf(cv[i], hs[j][i], yp);
                red[i] = l * dxj;               // dB[t, n]
                red[kGS + i] = dyj * hs[j][i];  // dC[t, n]
                mu[i] = a * l;
            }
            if constexpr (GZ) ypre[j] += yp;
            if (j == 0) {
                const float sum = wave_fold32(fold, sel8, sel4, sel2);
                if (stores && w.t0 + tk < L) part_l[kGS * g] = sum;
            }
#pragma unroll
            for (int i = 0; i < kGS; ++i) mu[i] = pin(mu[i]);
            ddt[j] = pin(ddt[j]); lbs[j] = pin(lbs[j]); ypre[j] = pin(ypre[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < kGS; ++i) s_acc[w.wave][kGS * g + i][w.lane] = dAacc[i];
    }

    // per token: skip, gate and step derivatives; stores
    float dD = 0.0f, dbias = 0.0f;
    float o_du[8], o_dr[8], o_dz[8];
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
        const float uj = ur.get(j);
        const bool in = w.t0 + j < L;
        o_du[j % 8] = fmaf(skip, dy[j], dt[j] * lbs[j]);
        const float dr = SP ? fmaf(uj, lbs[j], ddt[j]) * s_fin[w.wave][0][j][w.lane] : fmaf(uj, lbs[j], ddt[j]);
        o_dr[j % 8] = dr;
        if (in) {
            dD = fmaf(dy[j], uj, dD);
            dbias += dr;
        }
        if constexpr (GZ) {
            // dz = dout * y * SiLU'(z), y = readout + skip (zero past the end: dout is 0 there)
            o_dz[j % 8] = s_fin[w.wave][1][j][w.lane] * fmaf(skip, uj, ypre[j]);
        }
        if (j % 8 == 7 && w.active) {
            const int64_t tc0 = w.t0 + j - 7;
            store_chunk<IO, VEC>(static_cast<T*>(q.du) + w.row * L, tc0, L, o_du);
            store_chunk<IO, VEC>(static_cast<T*>(q.ddelta) + w.row * L, tc0, L, o_dr);
            if constexpr (GZ) store_chunk<IO, VEC>(static_cast<T*>(q.dz) + w.row * L, tc0, L, o_dz);
        }
    }
    s_acc[w.wave][kMaxState][w.lane] = dD;
    s_acc[w.wave][kMaxState + 1][w.lane] = dbias;
    __syncthreads();
    // the workgroup's 4 blocks summed; one partial per (batch row, segment, channel)
    if (w.wave == 0 && w.active) {
        const int64_t seg = w.blk / kWavesB;
        float* pa = q.dAp + ((w.b * q.nseg + seg) * q.a.nd + w.d) * kMaxState;
#pragma unroll
        for (int n = 0; n < kMaxState + 2; ++n) {
            const float v = ((s_acc[0][n][w.lane] + s_acc[1][n][w.lane]) + s_acc[2][n][w.lane]) + s_acc[3][n][w.lane];
            if (n < kMaxState) pa[n] = v;
            else if (n == kMaxState) q.dDp[(w.b * q.nseg + seg) * q.a.nd + w.d] = v;
            else q.dbp[(w.b * q.nseg + seg) * q.a.nd + w.d] = v;
        }
    }
}

// ---- 4. partial sums: dB, dC over channel groups; dA, dD, dbias over batch rows and segments
__global__ __launch_bounds__(256) void reduce_bc_kernel(BwdArgs q) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int N = q.a.N;
    const int64_t total = q.a.nb * q.a.L * N;
    if (gid >= total) return;
    const int n = static_cast<int>(gid % N);
    const int64_t bt = gid / N;  // b * L + t
    float sb = 0.0f, sc = 0.0f;
    const int64_t stride = q.a.nb * q.a.L * kMaxState;
    const float* pb = q.dBp + bt * kMaxState + n;
    const float* pc = q.dCp + bt * kMaxState + n;
    int64_t g = 0;
    for (; g + 4 <= q.groups; g += 4) {  // loads issued together; the sums keep their order
        const float b0 = pb[g * stride], b1 = pb[(g + 1) * stride], b2 = pb[(g + 2) * stride], b3 = pb[(g + 3) * stride];
        const float c0 = pc[g * stride], c1 = pc[(g + 1) * stride], c2 = pc[(g + 2) * stride], c3 = pc[(g + 3) * stride];
        sb = (((sb + b0) + b1) + b2) + b3;
        sc = (((sc + c0) + c1) + c2) + c3;
    }
    for (; g < q.groups; ++g) {
        sb += pb[g * stride];
        sc += pc[g * stride];
    }
    q.dB[gid] = sb;
    q.dC[gid] = sc;
}

__global__ __launch_bounds__(256) void reduce_channel_kernel(BwdArgs q) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int N = q.a.N;
    if (gid >= q.a.nd * (N + 2)) return;
    const int64_t d = gid / (N + 2);
    const int k = static_cast<int>(gid % (N + 2));
    // one strided series per lane: dA (stride nd * 16) or dD / dbias (stride nd)
    const float* src = k < N ? q.dAp + d * kMaxState + k : (k == N ? q.dDp : q.dbp) + d;
    const int64_t stride = k < N ? q.a.nd * kMaxState : q.a.nd;
    const int64_t cnt = q.a.nb * q.nseg;
    float s = 0.0f;
    int64_t bs = 0;
    for (; bs + 4 <= cnt; bs += 4) {  // loads issued together; the sum keeps its order
        const float v0 = src[bs * stride], v1 = src[(bs + 1) * stride], v2 = src[(bs + 2) * stride],
                    v3 = src[(bs + 3) * stride];
        s = (((s + v0) + v1) + v2) + v3;
    }
    for (; bs < cnt; ++bs) s += src[bs * stride];
    if (k < N) q.dA[d * N + k] = s;
    else if (k == N) { if (q.dD) q.dD[d] = s; }
    else if (q.dbias) q.dbias[d] = s;
}

template <typename IO, int NFIX, bool VEC, bool SP, bool GZ>
hipError_t launch_bwd_typed(const BwdArgs& q, hipStream_t s) {
    const uint32_t blocks = static_cast<uint32_t>(q.nbg * q.nseg);
    const int64_t lanes = q.nbg * kMaxState * 64;
    hipLaunchKernelGGL(segment_carry_kernel, dim3(static_cast<uint32_t>((lanes + 255) / 256)), dim3(256), 0, s, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((grad_kernel<IO, NFIX, VEC, SP, GZ>), dim3(blocks), dim3(kThreadsB), 0, s, q);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t nbc = q.a.nb * q.a.L * q.a.N;
    hipLaunchKernelGGL(reduce_bc_kernel, dim3(static_cast<uint32_t>((nbc + 255) / 256)), dim3(256), 0, s, q);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t nch = q.a.nd * (q.a.N + 2);
    hipLaunchKernelGGL(reduce_channel_kernel, dim3(static_cast<uint32_t>((nch + 255) / 256)), dim3(256), 0, s, q);
    return hipGetLastError();
}

template <typename IO, int NFIX, bool VEC>
hipError_t launch_bwd_flags(const BwdArgs& q, hipStream_t s) {
    const bool sp = q.a.softplus != 0, gz = q.a.z != nullptr;
    if (sp) return gz ? launch_bwd_typed<IO, NFIX, VEC, true, true>(q, s) : launch_bwd_typed<IO, NFIX, VEC, true, false>(q, s);
    return gz ? launch_bwd_typed<IO, NFIX, VEC, false, true>(q, s) : launch_bwd_typed<IO, NFIX, VEC, false, false>(q, s);
}

template <typename IO>
hipError_t launch_bwd_io(const BwdArgs& q, hipStream_t s) {
    const bool vec = q.a.L % (16 / IO::bytes) == 0;
    if (q.a.N == kMaxState)
        return vec ? launch_bwd_flags<IO, kMaxState, true>(q, s) : launch_bwd_flags<IO, kMaxState, false>(q, s);
    return vec ? launch_bwd_flags<IO, 0, true>(q, s) : launch_bwd_flags<IO, 0, false>(q, s);
}

}  // namespace

size_t scan_bwd_extra_bytes(int64_t nb, int64_t nd, int64_t L) {
    const int64_t nblk = ceil_div(L, kTok);
    const int64_t nseg = ceil_div(nblk, kWavesB);
    const int64_t groups = ceil_div(nd, 64);
    const int64_t rows = nb * nd;
    const int64_t floats = rows * nseg * kWavesB * kMaxState       // checkpoints
                           + groups * nb * nseg * kWavesB * 64 * (kMaxState + 1)  // block suffixes, step sums
                           + groups * nb * nseg * 64 * (2 * kMaxState + 1)  // segment aggregates and carries
                           + 2 * groups * nb * L * kMaxState       // dB, dC partials
                           + nb * nseg * nd * (kMaxState + 2);     // dA, dD, dbias partials
    return static_cast<size_t>(floats) * 4 + 16 * 256;             // + alignment slack
}

hipError_t launch_scan_bwd(BwdArgs q, bool io_bf16, void* scan_workspace, void* extra, hipStream_t s) {
    q.groups = (q.a.nd + 63) / 64;
    q.nbg = q.a.nb * q.groups;
    q.nblk = (q.a.L + kTok - 1) / kTok;
    q.nseg = (q.nblk + kWavesB - 1) / kWavesB;
    const int64_t rows = q.a.nb * q.a.nd;
    const int64_t cap = rows * q.nseg * kWavesB * kMaxState;  // blocks rounded up to whole segments
    auto carve = [&](size_t nfloats) {
        float* p = static_cast<float*>(extra);
        extra = static_cast<char*>(extra) + ((nfloats * 4 + 255) & ~size_t(255));
        return p;
    };
    float* hblk = carve(cap);
    q.hblk = hblk;
    q.lam = carve(q.nbg * q.nseg * kWavesB * kMaxState * 64);
    q.sdt = carve(q.nbg * q.nseg * kWavesB * 64);
    q.segagg = carve(q.nbg * q.nseg * (kMaxState + 1) * 64);
    q.segcarry = carve(q.nbg * q.nseg * kMaxState * 64);
    q.dBp = carve(q.groups * q.a.nb * q.a.L * kMaxState);
    q.dCp = carve(q.groups * q.a.nb * q.a.L * kMaxState);
    q.dAp = carve(q.a.nb * q.nseg * q.a.nd * kMaxState);
    q.dDp = carve(q.a.nb * q.nseg * q.a.nd);
    q.dbp = carve(q.a.nb * q.nseg * q.a.nd);
    // 1. the forward pass, writing only the block checkpoints, and the adjoint's block aggregates
    ScanArgs fa = q.a;
    fa.out = nullptr;
    fa.last_state = nullptr;
    fa.zoh = 0;
    fa.hblk = hblk;
    fa.dout = q.dout;
    fa.lam = q.lam;
    fa.sdt = q.sdt;
    fa.segagg = q.segagg;
    hipError_t e = launch_scan_ckpt(fa, io_bf16, scan_workspace, s);
    if (e != hipSuccess) return e;
    return io_bf16 ? launch_bwd_io<bf16_io>(q, s) : launch_bwd_io<f32_io>(q, s);
}

}  // namespace ssm
