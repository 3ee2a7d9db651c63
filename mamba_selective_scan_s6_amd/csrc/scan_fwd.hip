// scan_fwd.hip - selective scan forward (gfx950): one fused kernel, two sweeps per 64-token segment.
//
// Computes, per batch row b, channel d and token t ("Beyond attention with Mamba, state space
// models and hybrids", sections 3-4; "Module 19: State-Space Models (Mamba)", The Math):
//   Delta = softplus(delta + bias);  h_n = exp(Delta A_n) h_n + Delta B_{t,n} u;
//   y = sum_n C_{t,n} h_n + D u;  out = y * SiLU(z)
// The per-step states are never written to memory (section 6 of the first page: the fused kernel
// keeps them on chip and writes back only y).
//
// Parallel structure. The recurrence h_t = a_t h_{t-1} + b_t is a chain of affine maps, and
// composing two of them gives another, (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2) ("Module 19",
// The Parallel Scan). The sequence is cut into 64-token segments, one per workgroup:
//   * lanes = 64 consecutive channels of one batch row. B and C rows are the same for all of them:
//     each wave stages its tokens' rows in LDS (fp32) with one coalesced load per row block, and
//     every token reads its rows back as LDS broadcasts into ordinary VGPRs, so the per-state
//     arithmetic takes only VGPR operands (an SGPR or DPP operand halves the VALU rate on gfx950);
//   * each of the 4 waves owns 16 consecutive tokens of the segment for its 64 channels; u and z
//     stay in registers in the io format (bf16 two to a register), the steps Delta in fp32;
//   * pass A: every wave runs its 16 tokens from h = 0, giving its block's affine aggregate
//     (P_w, H_w), with P_w = 2^(a2 * sum of the block's steps);
//   * the waves' aggregates are combined through LDS into the segment aggregate, which is
//     published to a workspace; the segment then looks back at its predecessors (decoupled
//     look-back: fold published aggregates until a published inclusive state is found) to get
//     the state entering the segment, publishes its own inclusive state, and derives the state
//     entering each wave's block (these segment-level steps split the 16 states over the waves);
//   * pass B: each wave reruns its 16 tokens from that state, now with the readout, skip and gate,
//     and stores y 4 tokens at a time. Rerunning costs a second exponential per element-step but
//     holds no per-token state across the look-back, so a wave needs < 128 VGPRs and 16 waves
//     share a CU, which hides the load and look-back latency. 16 tokens per wave (not 8) halves
//     the number of workgroups, so the per-workgroup latency chain (loads, barriers, look-back,
//     publication) is paid half as often per token; it was measured 13-19% faster on the large
//     shapes.
// The ZOH template flag replaces the Euler input gain Delta B by the exact zero-order hold
// (e^{Delta A} - 1)/A B (zoh_gain); those variants hold 1/A per state and run 12 waves per CU.
// The OT template type is the output's element type: the input's, or fp32 when the caller asks for
// the value before its rounding to bf16. The CK variant is the backward's first pass: pass A, the
// look-back and the carries, writing the state entering every 16-token block, then the adjoint's pass
// over each block (its reverse aggregate), which needs the same block's steps and decays' arguments.
// Cross-workgroup data and flags use relaxed agent-scope atomics (coherent loads and stores);
// stores are ordered before the flag by waiting for their completion. Segments are assigned in
// segment-major workgroup order, so every segment depends only on lower workgroup indices. Every
// wait is bounded: on timeout the kernel records an error in the workspace header and goes on.
#include <atomic>

#include "lookback.hpp"
#include "scan_common.hpp"
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {
namespace {

using namespace scan;

constexpr int kWavesPerGroup = 4;  // waves per workgroup: a segment is 64 tokens of 64 channels
constexpr int kExpGroup = 4;       // decays computed back to back

template <typename OT>
struct OutIO;
template <>
struct OutIO<float> {
    using type = f32_io;
};
template <>
struct OutIO<uint16_t> {
    using type = bf16_io;
};
// Below this many channel groups (batch rows x 64-channel blocks) many consecutive segments of one
// group run at the same time: their look-backs start together, and a segment that published its
// aggregate only once its own look-back had to wait would cost every successor an extra round
// trip. Such shapes publish every aggregate at once (wave 1, while wave 0 polls); shapes with
// more groups publish lazily, which saves the workspace writes whenever the predecessor's
// inclusive state is already there. (Measured: 24 groups run faster eager; 32 groups, the
// long-context shape's, time the same either way, so they publish lazily.)
constexpr int64_t kEagerGroups = 32;
struct LbArgs {
    ScanArgs a;
    char* ws;         // workspace (lookback.hpp)
    int64_t groups;   // channel groups of 64 per batch row
    int64_t nbg;      // batch rows * groups
    int64_t S;        // segments per (batch row, group)
    uint32_t eager;   // publish every segment's aggregate at once (else only when its look-back waits)
    uint32_t vec;     // rows are read and written as 16-byte vectors (their length allows it)
    int spin_limit;   // polls a look-back may wait before it records a timeout
};

// IO: the input element type; OT: the output's (the input's, or fp32 with SSM_FLAG_OUT_F32). ZOH: the
// exact zero-order-hold input gain. CK: the backward's first pass (the state entering every 16-token
// block, no readout and no output; and the adjoint's pass over each block, which walks the same block).
template <int W, typename IO, typename OT, bool SP, bool GZ, bool ZOH, bool CK>
__global__ __launch_bounds__(W * 64, ZOH || CK ? 3 : 16 / W) void scan_fwd_kernel(LbArgs la) {
    constexpr int kWaves = W;                  // waves per workgroup, kTok consecutive tokens each
    constexpr int kSeg = kWaves * kTok;        // tokens per segment
    constexpr int kSPW = kMaxState / kWaves;   // states per wave in the segment-level steps
    constexpr int kFoldBatch = 16 / kSPW;      // predecessor aggregates loaded together in a fold
    using T = typename IO::storage;
    const ScanArgs& p = la.a;
    const uint64_t tag = lb::read_tag(la.ws);
    __shared__ float s_h[kWaves][kMaxState][64];  // per wave: H_w per state and lane; later the carry entering wave w
    __shared__ float s_sdt[kWaves][64];           // per wave: sum of the steps over its block
    __shared__ float s_hseg[kMaxState][64];       // the segment aggregate's H, per state and lane
    __shared__ __align__(16) float s_rows[kWaves][2][kTok][kMaxState];  // per wave: B and C rows of its tokens
    __shared__ int64_t s_jstar;

    // the wave index is uniform across a wave; saying so keeps per-wave addresses scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;

    const uint32_t item = blockIdx.x;
    // block counts fit in 32 bits (the library checks), so the index arithmetic stays 32-bit
    const uint32_t nbg32 = static_cast<uint32_t>(la.nbg), groups32 = static_cast<uint32_t>(la.groups);
    const uint32_t s32 = item / nbg32;  // segment index along the sequence
    const uint32_t bg32 = item - s32 * nbg32;
    const uint32_t b32 = bg32 / groups32;
    const int64_t s = s32, bg = bg32, b = b32;
    const int64_t d0 = static_cast<int64_t>(bg32 - b32 * groups32) * 64;  // first channel of the group
    const int64_t d = d0 + lane;
    const bool active = d < p.nd;
    const int64_t dc = active ? d : p.nd - 1;  // idle lanes compute on a valid row, store nothing
    const int N = p.N;
    const bool vec = la.vec != 0;
    const int64_t L = p.L;
    const int64_t S = la.S;
    const int64_t tw = s * kSeg + wave * kTok;  // first token of this wave's block

    const int64_t row = (b * p.nd + dc) * L;
    const T* __restrict__ Bb = static_cast<const T*>(p.B) + b * L * N;
    const T* __restrict__ Cb = static_cast<const T*>(p.C) + b * L * N;

    // ---- the segment's inputs. Every load is issued before any of them is used (the compiler waits for
    // a loaded value at its first use, in issue order), so the workgroup pays one memory round trip
    // before pass A instead of one per input: the B and C rows as raw words, bias and D, u and delta in
    // the io format, and A last (its 16 values per lane as four 16-byte loads when N = 16).
    const bool rows_fast = N == kMaxState && tw + kTok <= L;
    RowWords<IO> rbw, rcw;
    if (rows_fast) {
        fetch_rows<IO>(Bb, tw, lane, rbw);
        fetch_rows<IO>(Cb, tw, lane, rcw);
    }
    const float bias = p.delta_bias ? p.delta_bias[dc] : 0.0f;
    const float skip = p.D ? p.D[dc] : 0.0f;
    // u and z stay in the io format (the write scale Delta u and the skip term D u are formed where they
    // are used, one multiply each, instead of being held for every token); delta until its step is formed
    TokRow<IO> ur, zr, dr;
    if (vec) {
        load_tokrow<true>(static_cast<const T*>(p.u) + row, tw, L, ur);
        load_tokrow<true>(static_cast<const T*>(p.delta) + row, tw, L, dr);
    } else {
        load_tokrow<false>(static_cast<const T*>(p.u) + row, tw, L, ur);
        load_tokrow<false>(static_cast<const T*>(p.delta) + row, tw, L, dr);
    }
    float4 a4[kMaxState / 4];
    if (N == kMaxState) {
        const float4* ap = reinterpret_cast<const float4*>(p.A + dc * kMaxState);
#pragma unroll
        for (int k = 0; k < kMaxState / 4; ++k) a4[k] = ap[k];
    }

    // ---- B and C rows of this wave's tokens into LDS (fp32)
    if (rows_fast) {
        put_rows<IO>(rbw, lane, s_rows[wave][0]);
        put_rows<IO>(rcw, lane, s_rows[wave][1]);
    } else {
        stage_rows<IO, 0>(Bb, tw, L, N, lane, s_rows[wave][0]);
        stage_rows<IO, 0>(Cb, tw, L, N, lane, s_rows[wave][1]);
    }

    float a2[kMaxState];  // A * log2(e): exp(Delta A) = 2^(Delta a2)
    if (N == kMaxState) {
#pragma unroll
        for (int k = 0; k < kMaxState / 4; ++k) {
            a2[4 * k] = a4[k].x * kLog2e;
            a2[4 * k + 1] = a4[k].y * kLog2e;
            a2[4 * k + 2] = a4[k].z * kLog2e;
            a2[4 * k + 3] = a4[k].w * kLog2e;
        }
    } else {
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) a2[n] = n < N ? p.A[dc * N + n] * kLog2e : 0.0f;
    }
    float ia[ZOH ? kMaxState : 1];  // 1 / A for the zero-order-hold gain (unused where |Delta A| is small)
    if constexpr (ZOH) {
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) ia[n] = a2[n] != 0.0f ? kLog2e / a2[n] : 0.0f;
    }

    // ---- per-token steps
    float dt[kTok];
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
        const bool in = tw + j < L;
        const float r = dr.get(j) + bias;
        float st = r;
        if constexpr (SP) st = softplus_f32(r);
        dt[j] = in ? st : 0.0f;  // past the end: identity step (decay 1, no write)
    }

    // ---- pass A: the block's own state from h = 0 (its affine aggregate's H_w; P_w = 2^(a2 sum Delta))
    float h[kMaxState];
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) h[n] = 0.0f;
    {
        // each group of 4 states reads its 4 B values (one 16-byte LDS broadcast) one group ahead, so a
        // token never holds its whole row in registers
        float4 bn = read_quad(s_rows[wave][0][0], 0);
#pragma unroll
        for (int j = 0; j < kTok; ++j) {
            const float uj = pin(ur.get(j)), dtj = pin(dt[j]), dxj = dtj * uj;
#pragma unroll
            for (int g = 0; g < kMaxState; g += kExpGroup) {
                const float4 bq = bn;
                if (g + kExpGroup < kMaxState) bn = read_quad(s_rows[wave][0][j], (g + kExpGroup) / 4);
                else if (j + 1 < kTok) bn = read_quad(s_rows[wave][0][j + 1], 0);
                const float bk[kExpGroup] = {bq.x, bq.y, bq.z, bq.w};
                // the decays in groups of 4 ahead of the arithmetic that uses them: back-to-back
                // exponentials issue faster on this GPU than ones interleaved with other VALU work
                float yn[kExpGroup], an[kExpGroup];
#pragma unroll
                for (int k = 0; k < kExpGroup; ++k) {
                    yn[k] = dtj * a2[g + k];
                    an[k] = exp2_hw(yn[k]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 0; k < kExpGroup; ++k) {
                    const int n = g + k;
                    if constexpr (ZOH) h[n] = fmaf(an[k], h[n], bk[k] * (zoh_gain(yn[k], an[k], dtj, ia[n]) * uj));
                    else h[n] = fmaf(an[k], h[n], bk[k] * dxj);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // keep each token's work together: hoisting later tokens' exponentials would hold them all live
            pin_states(h);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    float sdt = 0.0f;
#pragma unroll
    for (int j = 0; j < kTok; ++j) sdt += dt[j];
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) s_h[wave][n][lane] = h[n];
    s_sdt[wave][lane] = sdt;
    __syncthreads();
    // the gate input, first used in pass B (with CK, dout and the gate input for the adjoint's pass): the
    // loads are in flight during the segment-level steps
    TokRow<IO> dor;
    if constexpr (GZ) {
        if (vec) load_tokrow<true>(static_cast<const T*>(p.z) + row, tw, L, zr);
        else load_tokrow<false>(static_cast<const T*>(p.z) + row, tw, L, zr);
    }
    if constexpr (CK) {
        if (vec) load_tokrow<true>(static_cast<const T*>(p.dout) + row, tw, L, dor);
        else load_tokrow<false>(static_cast<const T*>(p.dout) + row, tw, L, dor);
    }

    // ---- segment aggregate for this wave's kSPW states: the waves' blocks composed in token order
    float sw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sw[w] = s_sdt[w][lane];
    float sdt_seg = sw[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sdt_seg += sw[w];
    float hseg[kSPW], a2q[kSPW];
#pragma unroll
    for (int q = 0; q < kSPW; ++q) {
        const int n = kSPW * wave + q;
        a2q[q] = a2[n];
        float hq = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) hq = fmaf(exp2_hw(a2q[q] * sw[w]), hq, s_h[w][n][lane]);
        hseg[q] = hq;
    }
    const int64_t base = bg * S;  // this (batch row, group)'s slots
#pragma unroll
    for (int q = 0; q < kSPW; ++q) s_hseg[kSPW * wave + q][lane] = hseg[q];
    __syncthreads();

    // ---- decoupled look-back (wave 0): find the nearest predecessor with a published inclusive
    // state. In lazy mode the segment's aggregate is published only if the look-back has to wait; in
    // eager mode wave 1 publishes it at once, while wave 0 polls.
    auto publish_agg = [&]() {
        float* ag = lb::agg(la.ws, base + s);
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) lb::st(ag + n * 64 + lane, s_hseg[n][lane]);
        lb::st(ag + 16 * 64 + lane, sdt_seg);
        lb::wait_stores();
        if (lane == 0) lb::st_flag(lb::flag(la.ws, base + s), (tag << 2) | lb::kStatusAgg);
    };
    if (la.eager && wave == 1 && s > 0 && s < S - 1) {
        publish_agg();
        lb::wait_stores();
    }
    if (wave == 0) {
        int64_t jstar = -1;
        if (s > 0) jstar = lb::look_back(la.ws, base, s, tag, la.spin_limit, s == S - 1 || la.eager, publish_agg);
        if (lane == 0) {
            s_jstar = jstar;
            if (s == S - 1) lb::group_done(la.ws, tag, static_cast<uint32_t>(la.nbg));
        }
    }
    __syncthreads();

    // ---- fold: carry entering the segment for this wave's kSPW states
    const int64_t jstar = s_jstar;
    float c[kSPW];
#pragma unroll
    for (int q = 0; q < kSPW; ++q)
        c[q] = jstar >= 0 ? lb::ld(lb::incl(la.ws, base + jstar) + (kSPW * wave + q) * 64 + lane) : 0.0f;
    for (int64_t j0 = jstar + 1; j0 < s; j0 += kFoldBatch) {
        float hb[kFoldBatch][kSPW], sb[kFoldBatch];
#pragma unroll
        for (int k = 0; k < kFoldBatch; ++k) {
            const int64_t j = j0 + k < s ? j0 + k : s - 1;
            const float* ag = lb::agg(la.ws, base + j);
            sb[k] = lb::ld(ag + 16 * 64 + lane);
#pragma unroll
            for (int q = 0; q < kSPW; ++q) hb[k][q] = lb::ld(ag + (kSPW * wave + q) * 64 + lane);
        }
#pragma unroll
        for (int k = 0; k < kFoldBatch; ++k) {
            if (j0 + k < s) {
#pragma unroll
                for (int q = 0; q < kSPW; ++q) c[q] = fmaf(exp2_hw(a2q[q] * sb[k]), c[q], hb[k][q]);
            }
        }
    }

    // ---- inclusive state at the end of this segment; publish it, or write the final state
    float inc[kSPW];
#pragma unroll
    // The same arithmetic as a successor's fold of this segment's aggregate, fma(2^(a2 sum Delta),
    // carry, H): a carry then has the same bits whichever predecessor the look-back stopped at.
    for (int q = 0; q < kSPW; ++q) inc[q] = fmaf(exp2_hw(a2q[q] * sdt_seg), c[q], hseg[q]);
    if (s < S - 1) {
        float* ic = lb::incl(la.ws, base + s);
#pragma unroll
        for (int q = 0; q < kSPW; ++q) lb::st(ic + (kSPW * wave + q) * 64 + lane, inc[q]);
        lb::wait_stores();
    } else if (p.last_state && active) {
        float* st = p.last_state + (b * p.nd + d) * N;
#pragma unroll
        for (int q = 0; q < kSPW; ++q)
            if (kSPW * wave + q < N) st[kSPW * wave + q] = inc[q];
    }
    // carries entering each wave's block, for this wave's kSPW states (over H_w, which is read first)
#pragma unroll
    for (int q = 0; q < kSPW; ++q) {
        const int n = kSPW * wave + q;
        float v = c[q];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float hw = s_h[w][n][lane];
            s_h[w][n][lane] = v;
            v = fmaf(exp2_hw(a2q[q] * s_sdt[w][lane]), v, hw);  // the block's decay, recomputed (not held)
        }
    }
    __syncthreads();
    if (s < S - 1 && threadIdx.x == 0) lb::st_flag(lb::flag(la.ws, base + s), (tag << 2) | lb::kStatusIncl);

    if constexpr (!CK) {
        // ---- pass B: rerun the block from the state entering it; readout, skip, gate, store
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) h[n] = s_h[wave][n][lane];

        // Recomputing the decays and writes is cheaper than holding pass A's 2 x 128 values per lane
        // across the look-back; the opaque copies of the step and rows (pin) also keep the compiler from
        // merging the two passes' identical expressions.
        float o4[4];
        float4 bn = read_quad(s_rows[wave][0][0], 0), cn = read_quad(s_rows[wave][1][0], 0);
#pragma unroll
        for (int j = 0; j < kTok; ++j) {
            const float uj = ur.get(j);
            float acc0 = skip * uj, acc1 = 0.0f;
            const float dtj = pin(dt[j]), dxj = pin(dtj * uj);
#pragma unroll
            for (int g = 0; g < kMaxState; g += kExpGroup) {
                const float4 bq = bn, cq = cn;
                if (g + kExpGroup < kMaxState) {
                    bn = read_quad(s_rows[wave][0][j], (g + kExpGroup) / 4);
                    cn = read_quad(s_rows[wave][1][j], (g + kExpGroup) / 4);
                } else if (j + 1 < kTok) {
                    bn = read_quad(s_rows[wave][0][j + 1], 0);
                    cn = read_quad(s_rows[wave][1][j + 1], 0);
                }
                const float bk[kExpGroup] = {bq.x, bq.y, bq.z, bq.w}, ck[kExpGroup] = {cq.x, cq.y, cq.z, cq.w};
                float yn[kExpGroup], an[kExpGroup];
#pragma unroll
                for (int k = 0; k < kExpGroup; ++k) {
                    yn[k] = dtj * a2[g + k];
                    an[k] = exp2_hw(yn[k]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 0; k < kExpGroup; ++k) {
                    const int n = g + k;
                    if constexpr (ZOH) h[n] = fmaf(an[k], h[n], bk[k] * (zoh_gain(yn[k], an[k], dtj, ia[n]) * uj));
                    else h[n] = fmaf(an[k], h[n], bk[k] * dxj);
                    if (n & 1) acc1 = fmaf(ck[k], h[n], acc1);
                    else acc0 = fmaf(ck[k], h[n], acc0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            float out = acc0 + acc1;
            if constexpr (GZ) out *= silu_f32(zr.get(j));
            o4[j % 4] = pin(out);
            if (j % 4 == 3 && active) {
                using OIO = typename OutIO<OT>::type;
                if (vec) store_chunk4<OIO, true>(static_cast<OT*>(p.out) + row, tw + j - 3, L, o4);
                else store_chunk4<OIO, false>(static_cast<OT*>(p.out) + row, tw + j - 3, L, o4);
            }
            pin_states(h);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (CK && active && tw < L) {  // checkpoint for the backward pass: the state entering this block (in LDS)
        const int64_t nblk = (L + kTok - 1) / kTok;  // wave-uniform address part, then the lane's
        float* ckw = p.hblk + ((b * p.nd + d0) * nblk + tw / kTok) * kMaxState;
        float4* ck = reinterpret_cast<float4*>(ckw + static_cast<int64_t>(lane) * (nblk * kMaxState));
#pragma unroll
        for (int q = 0; q < kMaxState / 4; ++q)
            ck[q] = make_float4(s_h[wave][4 * q][lane], s_h[wave][4 * q + 1][lane], s_h[wave][4 * q + 2][lane],
                                s_h[wave][4 * q + 3][lane]);
    }
    if constexpr (CK) {
        // ---- the adjoint's pass over this block for the backward: from zero at the block's end,
        // mu <- exp(Delta A) (C dy + mu) backwards over its tokens (dy = dout SiLU(z)); mu after the
        // block's first decay and the block's sum of steps form its reverse aggregate
        float mu[kMaxState];
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) mu[n] = 0.0f;
#pragma unroll
        for (int j = kTok - 1; j >= 0; --j) {
            float cv[kMaxState];
            read_row(s_rows[wave][1][j], cv);
            float dy = dor.get(j);
            if constexpr (GZ) dy *= silu_f32(zr.get(j));
            const float dtj = pin(dt[j]), dyj = pin(dy);
#pragma unroll
            for (int n = 0; n < kMaxState; ++n) mu[n] = exp2_hw(dtj * a2[n]) * fmaf(cv[n], dyj, mu[n]);
            pin_states(mu);
            __builtin_amdgcn_sched_barrier(0);
        }
        // the blocks' reverse aggregates composed from zero at the segment's end (blocks past the
        // sequence's end compose as the identity: their steps and dout are zero), each wave composing
        // kSPW states: before each block, the suffix of the blocks after it in the segment (for the
        // gradient kernel's carry into that block), and at the end the segment's own aggregate (for the
        // carries between segments)
        __syncthreads();  // every wave has read its checkpoint from s_h
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) s_h[wave][n][lane] = mu[n];
        __syncthreads();
        float* sa = p.segagg + ((bg * S + s) * (kMaxState + 1)) * 64 + lane;
        float* sf = p.lam + (bg * S + s) * kWaves * kMaxState * 64 + lane;
#pragma unroll
        for (int q = 0; q < kSPW; ++q) {
            const int n = kSPW * wave + q;
            float m = 0.0f;
#pragma unroll
            for (int w = kWaves - 1; w >= 0; --w) {
                sf[(w * kMaxState + n) * 64] = m;
                m = fmaf(exp2_hw(a2q[q] * s_sdt[w][lane]), m, s_h[w][n][lane]);
            }
            sa[n * 64] = m;
        }
        if (wave == 0) sa[kMaxState * 64] = sdt_seg;
        // the step sum over the blocks after this wave's in the segment
        float ssuf = 0.0f;
#pragma unroll
        for (int w = kWaves - 1; w > 0; --w)
            if (w > wave) ssuf += s_sdt[w][lane];
        p.sdt[((bg * S + s) * kWaves + wave) * 64 + lane] = ssuf;
    }
}

template <int W, typename IO, typename OT, bool SP, bool GZ, bool ZOH, bool CK>
hipError_t launch_typed(const LbArgs& la, hipStream_t s) {
    const int64_t blocks = la.nbg * la.S;
    hipLaunchKernelGGL((scan_fwd_kernel<W, IO, OT, SP, GZ, ZOH, CK>), dim3(static_cast<uint32_t>(blocks)), dim3(W * 64),
                       0, s, la);
    return hipGetLastError();
}

template <int W, typename IO, typename OT, bool ZOH>
hipError_t launch_flags(const LbArgs& la, hipStream_t s) {
    const bool sp = la.a.softplus != 0, gz = la.a.z != nullptr;
    if (sp) return gz ? launch_typed<W, IO, OT, true, true, ZOH, false>(la, s) : launch_typed<W, IO, OT, true, false, ZOH, false>(la, s);
    return gz ? launch_typed<W, IO, OT, false, true, ZOH, false>(la, s) : launch_typed<W, IO, OT, false, false, ZOH, false>(la, s);
}

template <int W, typename IO, typename OT>
hipError_t launch_zoh(const LbArgs& la, hipStream_t s) {
    return la.a.zoh ? launch_flags<W, IO, OT, true>(la, s) : launch_flags<W, IO, OT, false>(la, s);
}

int64_t segments(int64_t L, int seg) { return ceil_div(L, seg); }

LbArgs make_args(const ScanArgs& a, bool io_bf16, void* workspace) {
    LbArgs la;
    la.a = a;
    la.ws = static_cast<char*>(workspace);
    la.groups = ceil_div(a.nd, 64);
    la.nbg = a.nb * la.groups;
    la.S = segments(a.L, kWavesPerGroup * kTok);
    la.eager = la.nbg < kEagerGroups ? 1u : 0u;
    // 16-byte vectors along a row need its length in elements to be a multiple of 16 bytes (the
    // tensors themselves are 16-byte aligned); an fp32 output of bf16 inputs needs it for both
    la.vec = a.L % (16 / (io_bf16 ? 2 : 4)) == 0 && (!a.out_f32 || a.L % 4 == 0) ? 1u : 0u;
    la.spin_limit = scan_wait_limit();
    return la;
}

std::atomic<int> g_spin_limit{lb::kDefaultSpinLimit};

}  // namespace

size_t scan_workspace_bytes(int64_t nb, int64_t nd, int64_t L) {
    return lb::workspace_bytes(nb * ceil_div(nd, 64) * segments(L, kWavesPerGroup * kTok));
}

int64_t scan_max_blocks(int64_t nb, int64_t nd, int64_t L) {
    return sat_mul(sat_mul(nb, ceil_div(nd, 64)), segments(L, kWavesPerGroup * kTok));
}

int scan_segment_tokens(int64_t, int64_t, int64_t) { return kWavesPerGroup * kTok; }

int set_scan_wait_limit(int polls) { return g_spin_limit.exchange(polls > 0 ? polls : lb::kDefaultSpinLimit); }

int scan_wait_limit() { return g_spin_limit.load(std::memory_order_relaxed); }

hipError_t launch_scan_fwd(const ScanArgs& a, bool io_bf16, void* workspace, hipStream_t s) {
    constexpr int W = kWavesPerGroup;
    const LbArgs la = make_args(a, io_bf16, workspace);
    if (!io_bf16) return launch_zoh<W, f32_io, float>(la, s);
    return a.out_f32 ? launch_zoh<W, bf16_io, float>(la, s) : launch_zoh<W, bf16_io, uint16_t>(la, s);
}

// The backward's first pass: Euler input gain, no readout, no output; the checkpoints and the adjoint's
// block aggregates (GZ: the gate's SiLU(z) scales dout).
template <typename IO>
hipError_t launch_ckpt_io(const LbArgs& la, hipStream_t s) {
    constexpr int W = kWavesPerGroup;
    const bool sp = la.a.softplus != 0, gz = la.a.z != nullptr;
    if (sp) return gz ? launch_typed<W, IO, float, true, true, false, true>(la, s)
                      : launch_typed<W, IO, float, true, false, false, true>(la, s);
    return gz ? launch_typed<W, IO, float, false, true, false, true>(la, s)
              : launch_typed<W, IO, float, false, false, false, true>(la, s);
}

hipError_t launch_scan_ckpt(const ScanArgs& a, bool io_bf16, void* workspace, hipStream_t s) {
    const LbArgs la = make_args(a, io_bf16, workspace);
    return io_bf16 ? launch_ckpt_io<bf16_io>(la, s) : launch_ckpt_io<f32_io>(la, s);
}

}  // namespace ssm
