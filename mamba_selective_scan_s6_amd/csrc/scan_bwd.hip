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
//   1. the forward kernel in checkpoint mode writes the state entering each 16-token block;
//   2. adjoint_block_kernel: per block, the adjoint from zero at the block's end; its value after
//      the block's first decay (mu = a_first lambda_first) and the block's decay 2^(a2 sum Delta)
//      form the block's affine aggregate, as in the forward pass but in reverse;
//   3. adjoint_carry_kernel: per (channel, state), the carries into every block from the right,
//      composing those aggregates from the end of the sequence;
//   4. grad_kernel: per block, the states recomputed from the checkpoint (2 states at a time, the
//      16 tokens kept in registers), then the adjoint backwards through the block with every
//      gradient term; the sums over channels (dB, dC) go through LDS into per-group partials, the
//      sums over tokens (dA, dD, dbias) into per-workgroup partials;
//   5. reduce_bc_kernel, reduce_channel_kernel: the partials summed into the outputs.
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
static_assert(kNV == 4, "the transpose reads one float4 per lane and sums along 16-lane rows");

// d SiLU(z) / dz = sigmoid(z) (1 + z (1 - sigmoid(z)))
__device__ __forceinline__ float dsilu_f32(float z) {
    const float sg = __builtin_amdgcn_rcpf(1.0f + exp2_hw(-z * kLog2e));
    return sg * fmaf(z, 1.0f - sg, 1.0f);
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

// Step Delta (0 past the end) and, with softplus, its derivative sigmoid(r) for one wave's tokens.
template <typename IO, bool VEC, bool SP>
__device__ __forceinline__ void load_steps(const BwdArgs& q, const WaveIdx& w, float (&dt)[kTok], float (&dsp)[kTok]) {
    using T = typename IO::storage;
    float rr[kTok];
    load_block<IO, VEC>(static_cast<const T*>(q.a.delta) + w.row * q.a.L, w.t0, q.a.L, rr);
    const float bias = q.a.delta_bias ? q.a.delta_bias[w.dc] : 0.0f;
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
        const float r = rr[j] + bias;
        const bool in = w.t0 + j < q.a.L;
        dt[j] = in ? (SP ? softplus_f32(r) : r) : 0.0f;
        dsp[j] = SP ? __builtin_amdgcn_rcpf(1.0f + exp2_hw(-r * kLog2e)) : 1.0f;
    }
}

// dy = dout * SiLU(z) (dout alone without a gate); zero past the end.
template <typename IO, bool VEC, bool GZ>
__device__ __forceinline__ void load_dy(const BwdArgs& q, const WaveIdx& w, float (&dy)[kTok]) {
    using T = typename IO::storage;
    load_block<IO, VEC>(static_cast<const T*>(q.dout) + w.row * q.a.L, w.t0, q.a.L, dy);
    if constexpr (GZ) {
        float zz[kTok];
        load_block<IO, VEC>(static_cast<const T*>(q.a.z) + w.row * q.a.L, w.t0, q.a.L, zz);
#pragma unroll
        for (int j = 0; j < kTok; ++j) dy[j] *= silu_f32(zz[j]);
    }
}

// ---- 2. reverse aggregate of each block: mu after the block's first decay, from zero at its end
template <typename IO, int NFIX, bool VEC, bool SP, bool GZ>
__global__ __launch_bounds__(kThreadsB) void adjoint_block_kernel(BwdArgs q) {
    __shared__ __align__(16) float s_rows[kWavesB][kTok][kMaxState];
    const WaveIdx w = wave_index(q);
    const int N = NFIX == kMaxState ? kMaxState : q.a.N;
    using T = typename IO::storage;
    stage_rows<IO, NFIX>(static_cast<const T*>(q.a.C) + w.b * q.a.L * N, w.t0, q.a.L, N, w.lane, s_rows[w.wave]);
    float dt[kTok], dsp[kTok], dy[kTok];
    load_steps<IO, VEC, SP>(q, w, dt, dsp);
    load_dy<IO, VEC, GZ>(q, w, dy);
    float a2[kMaxState];
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) a2[n] = n < N ? q.a.A[w.dc * N + n] * kLog2e : 0.0f;
    float mu[kMaxState];
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) mu[n] = 0.0f;
#pragma unroll
    for (int j = kTok - 1; j >= 0; --j) {
        float cv[kMaxState];
        read_row(s_rows[w.wave][j], cv);
        const float dtj = pin(dt[j]), dyj = pin(dy[j]);
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) mu[n] = exp2_hw(dtj * a2[n]) * fmaf(cv[n], dyj, mu[n]);
        pin_states(mu);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (w.active && w.t0 < q.a.L) {
        float4* dst = reinterpret_cast<float4*>(q.lam + (w.row * q.nblk + w.blk) * kMaxState);
#pragma unroll
        for (int k = 0; k < kMaxState / 4; ++k) dst[k] = make_float4(mu[4 * k], mu[4 * k + 1], mu[4 * k + 2], mu[4 * k + 3]);
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < kTok; ++j) s += dt[j];
        q.sdt[w.row * q.nblk + w.blk] = s;
    }
}

// ---- 3. carries into each block from the right: one lane per (batch row, channel, state)
__global__ __launch_bounds__(256) void adjoint_carry_kernel(BwdArgs q) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= q.a.nb * q.a.nd * kMaxState) return;
    const int n = static_cast<int>(gid % kMaxState);
    const int64_t row = gid / kMaxState;
    const int64_t d = row % q.a.nd;
    const int N = q.a.N;
    const float a2 = n < N ? q.a.A[d * N + n] * kLog2e : 0.0f;
    const float* lam = q.lam + row * q.nblk * kMaxState + n;
    const float* sdt = q.sdt + row * q.nblk;
    float* muin = q.muin + row * q.nblk * kMaxState + n;
    float mu = 0.0f;  // nothing enters the last block from the right
    int64_t k = q.nblk - 1;
    constexpr int kU = 8;  // blocks whose loads are issued together (the chain through mu stays serial)
    for (; k >= kU - 1; k -= kU) {
        float lv[kU], sv[kU];
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            lv[i] = lam[(k - i) * kMaxState];
            sv[i] = sdt[k - i];
        }
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            muin[(k - i) * kMaxState] = mu;
            mu = fmaf(exp2_hw(a2 * sv[i]), mu, lv[i]);
        }
    }
    for (; k >= 0; --k) {
        muin[k * kMaxState] = mu;
        mu = fmaf(exp2_hw(a2 * sdt[k]), mu, lam[k * kMaxState]);
    }
}

// ---- 4. gradients of one block
template <typename IO, int NFIX, bool VEC, bool SP, bool GZ>
__global__ __launch_bounds__(kThreadsB, 2) void grad_kernel(BwdArgs q) {
    using T = typename IO::storage;
    __shared__ __align__(16) float s_rows[kWavesB][2][kTok][kMaxState];
    __shared__ __align__(16) float s_red[kWavesB][kNV][64];  // one token's dB, dC partials of kGS states
    __shared__ float s_acc[kWavesB][kMaxState + 2][64];  // per wave: dA (16 states), dD, dbias
    const WaveIdx w = wave_index(q);
    const int N = NFIX == kMaxState ? kMaxState : q.a.N;
    const int64_t L = q.a.L;
    stage_rows<IO, NFIX>(static_cast<const T*>(q.a.B) + w.b * L * N, w.t0, L, N, w.lane, s_rows[w.wave][0]);
    stage_rows<IO, NFIX>(static_cast<const T*>(q.a.C) + w.b * L * N, w.t0, L, N, w.lane, s_rows[w.wave][1]);

    float dt[kTok], dsp[kTok], dy[kTok];
    load_steps<IO, VEC, SP>(q, w, dt, dsp);
    load_dy<IO, VEC, GZ>(q, w, dy);
    TokRow<IO> ur;
    load_tokrow<VEC>(static_cast<const T*>(q.a.u) + w.row * L, w.t0, L, ur);
    const float skip = q.a.D ? q.a.D[w.dc] : 0.0f;

    float ddt[kTok], dux[kTok], ypre[kTok];
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
        ddt[j] = 0.0f;
        dux[j] = 0.0f;
        ypre[j] = 0.0f;
    }
    // a block past the end reads the last block's checkpoint and carry (valid memory); with zero steps,
    // dy and u it adds exactly nothing
    const int64_t blk_r = w.blk < q.nblk ? w.blk : q.nblk - 1;
    const float* hin = q.hblk + (w.row * q.nblk + blk_r) * kMaxState;
    const float* muin = q.muin + (w.row * q.nblk + blk_r) * kMaxState;
    // per-lane transpose slot for the dB / dC sums: lane -> (value tv, chunk tc of kNV channels)
    constexpr int kLV = 64 / kNV;  // lanes per value
    const int tv = w.lane / kLV, tc = w.lane % kLV;

#pragma unroll 1
    for (int g = 0; g < kMaxState / kGS; ++g) {  // kGS states at a time
        float a2[kGS], h0[kGS], mu[kGS], dAacc[kGS];
#pragma unroll
        for (int i = 0; i < kGS; ++i) {
            const int n = kGS * g + i;
            a2[i] = n < N ? q.a.A[w.dc * N + n] * kLog2e : 0.0f;
            h0[i] = hin[n];
            mu[i] = muin[n];
            dAacc[i] = 0.0f;
        }
        // forward: the states of the block's 16 tokens for these kGS states
        float hs[kTok][kGS];
#pragma unroll
        for (int j = 0; j < kTok; ++j) {
            const float dtj = pin(dt[j]), dxj = dtj * pin(ur.get(j));
            const float2 bq = *reinterpret_cast<const float2*>(&s_rows[w.wave][0][j][kGS * g]);
            const float bv[kGS] = {bq.x, bq.y};
#pragma unroll
            for (int i = 0; i < kGS; ++i) {
                const float prev = j > 0 ? hs[j - 1][i] : h0[i];
                hs[j][i] = pin(fmaf(exp2_hw(dtj * a2[i]), prev, bv[i] * dxj));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // backward through the block
#pragma unroll
        for (int j = kTok - 1; j >= 0; --j) {
            const float uj = pin(ur.get(j)), dtj = pin(dt[j]), dyj = pin(dy[j]);
            const float2 bq = *reinterpret_cast<const float2*>(&s_rows[w.wave][0][j][kGS * g]);
            const float2 cq = *reinterpret_cast<const float2*>(&s_rows[w.wave][1][j][kGS * g]);
            const float bv[kGS] = {bq.x, bq.y}, cv[kGS] = {cq.x, cq.y};
            float red[kNV];
#pragma unroll
            for (int i = 0; i < kGS; ++i) {
                const float l = fmaf(cv[i], dyj, mu[i]);
                const float a = exp2_hw(dtj * a2[i]);
                const float hp = j > 0 ? hs[j - 1][i] : h0[i];
                const float ha = hp * a;
                ddt[j] = fmaf(l, fmaf(ha, a2[i] * kLn2, bv[i] * uj), ddt[j]);
                dux[j] = fmaf(l * dtj, bv[i], dux[j]);
                dAacc[i] = fmaf(l * ha, dtj, dAacc[i]);
                ypre[j] = fmaf(cv[i], hs[j][i], ypre[j]);
                red[i] = l * dtj * uj;  // dB[t, n]
                red[kGS + i] = dyj * hs[j][i];  // dC[t, n]
                mu[i] = a * l;
            }
            // sums over the wave's 64 channels: transpose through LDS, kLV = 16 lanes (one DPP row) per
            // value, each lane adding kNV channels, then a prefix sum along the row
#pragma unroll
            for (int v = 0; v < kNV; ++v) s_red[w.wave][v][w.lane] = w.active ? red[v] : 0.0f;
            const float4 pv = *reinterpret_cast<const float4*>(&s_red[w.wave][tv][kNV * tc]);
            float sum = (pv.x + pv.y) + (pv.z + pv.w);
            // prefix sum along the 16-lane row (DPP row_shr 1, 2, 4, 8): its last lane gets the total
            sum += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sum), 0x111, 0xf, 0xf, true));
            sum += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sum), 0x112, 0xf, 0xf, true));
            sum += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sum), 0x114, 0xf, 0xf, true));
            sum += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sum), 0x118, 0xf, 0xf, true));
            const int64_t t = w.t0 + j;
            if (tc == kLV - 1 && t < L) {
                float* part = (tv < kGS ? q.dBp : q.dCp) + ((w.d0 / 64 * q.a.nb + w.b) * L + t) * kMaxState;
                part[kGS * g + (tv % kGS)] = sum;
            }
#pragma unroll
            for (int i = 0; i < kGS; ++i) mu[i] = pin(mu[i]);
            ddt[j] = pin(ddt[j]); dux[j] = pin(dux[j]); ypre[j] = pin(ypre[j]);
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
        o_du[j % 8] = fmaf(skip, dy[j], dux[j]);
        const float dr = ddt[j] * dsp[j];
        o_dr[j % 8] = dr;
        if (in) {
            dD = fmaf(dy[j], uj, dD);
            dbias += dr;
        }
        if constexpr (GZ) {
            // dz = dout * y * SiLU'(z), y = readout + skip; dout and z are re-read (cheap: cached lines)
            const float dj = in ? load_elem(static_cast<const T*>(q.dout), w.row * L + w.t0 + j) : 0.0f;
            const float zj = in ? load_elem(static_cast<const T*>(q.a.z), w.row * L + w.t0 + j) : 0.0f;
            o_dz[j % 8] = dj * fmaf(skip, uj, ypre[j]) * dsilu_f32(zj);
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

// ---- 5. partial sums: dB, dC over channel groups; dA, dD, dbias over batch rows and segments
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
    hipLaunchKernelGGL((adjoint_block_kernel<IO, NFIX, VEC, SP, GZ>), dim3(blocks), dim3(kThreadsB), 0, s, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t lanes = q.a.nb * q.a.nd * kMaxState;
    hipLaunchKernelGGL(adjoint_carry_kernel, dim3(static_cast<uint32_t>((lanes + 255) / 256)), dim3(256), 0, s, q);
    if ((e = hipGetLastError()) != hipSuccess) return e;
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
    const int64_t nblk = (L + kTok - 1) / kTok;
    const int64_t nseg = (nblk + kWavesB - 1) / kWavesB;
    const int64_t groups = (nd + 63) / 64;
    const int64_t rows = nb * nd;
    const int64_t floats = 3 * rows * nseg * kWavesB * kMaxState  // checkpoints, block aggregates, carries
                           + rows * nseg * kWavesB                 // block step sums
                           + 2 * groups * nb * L * kMaxState       // dB, dC partials
                           + nb * nseg * nd * (kMaxState + 2);     // dA, dD, dbias partials
    return static_cast<size_t>(floats) * 4 + 16 * 256;             // + alignment slack
}

hipError_t launch_scan_bwd(BwdArgs q, bool io_bf16, void* scan_workspace, uint32_t epoch, void* extra, hipStream_t s) {
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
    q.lam = carve(cap);
    q.muin = carve(cap);
    q.sdt = carve(rows * q.nseg * kWavesB);
    q.dBp = carve(q.groups * q.a.nb * q.a.L * kMaxState);
    q.dCp = carve(q.groups * q.a.nb * q.a.L * kMaxState);
    q.dAp = carve(q.a.nb * q.nseg * q.a.nd * kMaxState);
    q.dDp = carve(q.a.nb * q.nseg * q.a.nd);
    q.dbp = carve(q.a.nb * q.nseg * q.a.nd);
    // 1. the forward pass, writing only the block checkpoints
    ScanArgs fa = q.a;
    fa.out = nullptr;
    fa.last_state = nullptr;
    fa.zoh = 0;
    fa.hblk = hblk;
    hipError_t e = launch_scan_fwd(fa, io_bf16, scan_workspace, epoch, s);
    if (e != hipSuccess) return e;
    return io_bf16 ? launch_bwd_io<bf16_io>(q, s) : launch_bwd_io<f32_io>(q, s);
}

}  // namespace ssm
