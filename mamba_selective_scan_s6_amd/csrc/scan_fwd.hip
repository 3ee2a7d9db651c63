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
//     and stores y 8 tokens at a time. Rerunning costs a second exponential per element-step but
//     holds no per-token state across the look-back, so a wave needs < 128 VGPRs and 16 waves
//     share a CU, which hides the load and look-back latency. 16 tokens per wave (not 8) halves
//     the number of workgroups, so the per-workgroup latency chain (loads, barriers, look-back,
//     publication) is paid half as often per token; it was measured 13-19% faster on the large
//     shapes.
// The ZOH template flag replaces the Euler input gain Delta B by the exact zero-order hold
// (e^{Delta A} - 1)/A B (zoh_gain); those variants hold 1/A per state and run 12 waves per CU.
// Cross-workgroup data and flags use relaxed agent-scope atomics (coherent loads and stores);
// stores are ordered before the flag by waiting for their completion. Segments are assigned in
// segment-major workgroup order, so every segment depends only on lower workgroup indices. Every
// wait is bounded: on timeout the kernel records an error in the workspace header and goes on.
#include <atomic>

#include "scan_common.hpp"
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {
namespace {

using namespace scan;

constexpr int kWavesPerGroup = 4;  // waves per workgroup: a segment is 64 tokens of 64 channels
// Below this many channel groups (batch rows x 64-channel blocks) many consecutive segments of one
// group run at the same time: their look-backs start together, and a segment that published its
// aggregate only once its own look-back had to wait would cost every successor an extra round
// trip. Such shapes publish every aggregate at once (wave 1, while wave 0 polls); shapes with
// more groups publish lazily, which saves the workspace writes whenever the predecessor's
// inclusive state is already there.
constexpr int64_t kEagerGroups = 128;
constexpr uint32_t kStatusAgg = 1;
constexpr uint32_t kStatusIncl = 2;
constexpr int kSpinLimit = 200000;  // default wait: polls (each with a short sleep), about 0.1 s
std::atomic<int> g_spin_limit{kSpinLimit};

struct LbArgs {
    ScanArgs a;
    int64_t groups;  // channel groups of 64 per batch row
    int64_t nbg;     // batch rows * groups
    int64_t S;       // segments per (batch row, group)
    uint32_t epoch;  // tag of this launch in the workspace flags (30 bits)
    uint32_t* flags;  // [nbg * S]
    float* agg;       // [nbg * S][17][64]: H for 16 states, then the segment's sum of Delta
    float* incl;      // [nbg * S][16][64]: state at the end of the segment
    uint32_t* error;  // workspace header word
    uint32_t eager;   // publish every segment's aggregate at once (else only when its look-back waits)
    int spin_limit;   // polls a look-back may wait before it records a timeout
};

__device__ __forceinline__ float ld_coherent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_flag(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int W, typename IO, int NFIX, bool VEC, bool SP, bool GZ, bool ZOH, bool CK>
__global__ __launch_bounds__(W * 64, ZOH || CK ? 3 : 16 / W) void scan_fwd_kernel(LbArgs lb) {
    constexpr int kWaves = W;                  // waves per workgroup, 8 consecutive tokens each
    constexpr int kSeg = kWaves * kTok;        // tokens per segment
    constexpr int kSPW = kMaxState / kWaves;   // states per wave in the segment-level steps
    constexpr int kFoldBatch = 16 / kSPW;      // predecessor aggregates loaded together in a fold
    using T = typename IO::storage;
    const ScanArgs& p = lb.a;
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
    const uint32_t nbg32 = static_cast<uint32_t>(lb.nbg), groups32 = static_cast<uint32_t>(lb.groups);
    const uint32_t s32 = item / nbg32;  // segment index along the sequence
    const uint32_t bg32 = item - s32 * nbg32;
    const uint32_t b32 = bg32 / groups32;
    const int64_t s = s32, bg = bg32, b = b32;
    const int64_t d0 = static_cast<int64_t>(bg32 - b32 * groups32) * 64;  // first channel of the group
    const int64_t d = d0 + lane;
    const bool active = d < p.nd;
    const int64_t dc = active ? d : p.nd - 1;  // idle lanes compute on a valid row, store nothing
    const int N = NFIX == kMaxState ? kMaxState : p.N;
    const int64_t L = p.L;
    const int64_t S = lb.S;
    const int64_t tw = s * kSeg + wave * kTok;  // first token of this wave's block

    const int64_t row = (b * p.nd + dc) * L;
    const T* __restrict__ Bb = static_cast<const T*>(p.B) + b * L * N;
    const T* __restrict__ Cb = static_cast<const T*>(p.C) + b * L * N;

    // ---- B and C rows of this wave's tokens into LDS (fp32)
    stage_rows<IO, NFIX>(Bb, tw, L, N, lane, s_rows[wave][0]);
    stage_rows<IO, NFIX>(Cb, tw, L, N, lane, s_rows[wave][1]);

    float a2[kMaxState];  // A * log2(e): exp(Delta A) = 2^(Delta a2)
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) a2[n] = n < N ? p.A[dc * N + n] * kLog2e : 0.0f;
    float ia[ZOH ? kMaxState : 1];  // 1 / A for the zero-order-hold gain (unused where |Delta A| is small)
    if constexpr (ZOH) {
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) ia[n] = a2[n] != 0.0f ? kLog2e / a2[n] : 0.0f;
    }
    const float bias = p.delta_bias ? p.delta_bias[dc] : 0.0f;
    const float skip = p.D ? p.D[dc] : 0.0f;

    // ---- per-token quantities: step, write scale, skip term (the readout starts from it), gate input
    // (u and z stay in the io format; the write scale Delta u and the skip term D u are formed where
    // they are used, one multiply each, instead of being held for every token)
    float dt[kTok];
    TokRow<IO> ur, zr;
    {
        float rr[kTok];
        load_tokrow<VEC>(static_cast<const T*>(p.u) + row, tw, L, ur);
        load_block<IO, VEC>(static_cast<const T*>(p.delta) + row, tw, L, rr);
        if constexpr (GZ) load_tokrow<VEC>(static_cast<const T*>(p.z) + row, tw, L, zr);
#pragma unroll
        for (int j = 0; j < kTok; ++j) {
            const bool in = tw + j < L;
            const float r = rr[j] + bias;
            float st = r;
            if constexpr (SP) st = softplus_f32(r);
            dt[j] = in ? st : 0.0f;  // past the end: identity step (decay 1, no write)
        }
    }

    // ---- pass A: the block's own state from h = 0 (its affine aggregate's H_w; P_w = 2^(a2 sum Delta))
    float h[kMaxState];
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) h[n] = 0.0f;
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
        const float uj = pin(ur.get(j)), dtj = pin(dt[j]), dxj = dtj * uj;
        float bv[kMaxState];
        read_row(s_rows[wave][0][j], bv);
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) {
            const float yn = dtj * a2[n], an = exp2_hw(yn);
            if constexpr (ZOH) h[n] = fmaf(an, h[n], bv[n] * (zoh_gain(yn, an, dtj, ia[n]) * uj));
            else h[n] = fmaf(an, h[n], bv[n] * dxj);
        }
        // keep each token's work together: hoisting later tokens' exponentials would hold them all live
        pin_states(h);
        __builtin_amdgcn_sched_barrier(0);
    }
    float sdt = 0.0f;
#pragma unroll
    for (int j = 0; j < kTok; ++j) sdt += dt[j];
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) s_h[wave][n][lane] = h[n];
    s_sdt[wave][lane] = sdt;
    __syncthreads();

    // ---- segment aggregate for this wave's kSPW states: the waves' blocks composed in token order
    float sw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sw[w] = s_sdt[w][lane];
    float sdt_seg = sw[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sdt_seg += sw[w];
    float hseg[kSPW], a2q[kSPW], pw[kSPW][kWaves];
#pragma unroll
    for (int q = 0; q < kSPW; ++q) {
        const int n = kSPW * wave + q;
        a2q[q] = a2[n];
        float hq = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            pw[q][w] = exp2_hw(a2q[q] * sw[w]);
            hq = fmaf(pw[q][w], hq, s_h[w][n][lane]);
        }
        hseg[q] = hq;
    }
    const int64_t base = bg * S;  // this (batch row, group)'s slots
    const uint32_t tag = lb.epoch << 2;
#pragma unroll
    for (int q = 0; q < kSPW; ++q) s_hseg[kSPW * wave + q][lane] = hseg[q];
    __syncthreads();

    // ---- decoupled look-back (wave 0): find the nearest predecessor with a published inclusive
    // state. In lazy mode the segment's aggregate is published only if the look-back has to wait: a
    // segment whose carry resolves at once publishes its inclusive state soon after, and the
    // aggregate would be workspace traffic that no successor reads. In eager mode wave 1 publishes
    // it at once, while wave 0 polls.
    if (lb.eager && wave == 1 && s > 0 && s < S - 1) {  // eager publication, beside wave 0's look-back
        float* ag = lb.agg + (base + s) * (17 * 64);
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) st_coherent(ag + n * 64 + lane, s_hseg[n][lane]);
        st_coherent(ag + 16 * 64 + lane, sdt_seg);
        __builtin_amdgcn_s_waitcnt(0);
        if (lane == 0) st_flag(lb.flags + base + s, tag | kStatusAgg);
        __builtin_amdgcn_s_waitcnt(0);  // the flag lands before this segment's inclusive flag can
    }
    if (wave == 0) {
        int64_t jstar = -1;
        if (s > 0) {
            int64_t jhi = s - 1;
            int spins = 0;
            bool published = s == S - 1 || lb.eager;  // the last segment has no successor
            for (;;) {
                const int64_t j = jhi - lane;  // lane 0 = nearest predecessor
                uint32_t st = kStatusIncl;     // j < 0: the zero initial state counts as inclusive
                if (j >= 0) {
                    const uint32_t f = ld_flag(lb.flags + base + j);
                    st = (f & ~3u) == tag ? (f & 3u) : 0u;
                }
                const uint64_t incl_mask = __ballot(st == kStatusIncl);
                const uint64_t none_mask = __ballot(st == 0u);
                const int first = incl_mask ? __builtin_ctzll(incl_mask) : 64;
                const uint64_t before = first >= 64 ? ~0ull : ((1ull << first) - 1ull);
                if (none_mask & before) {  // a predecessor has not published yet: wait
                    if (!published) {  // first let successors fold past this segment
                        float* ag = lb.agg + (base + s) * (17 * 64);
#pragma unroll
                        for (int n = 0; n < kMaxState; ++n) st_coherent(ag + n * 64 + lane, s_hseg[n][lane]);
                        st_coherent(ag + 16 * 64 + lane, sdt_seg);
                        __builtin_amdgcn_s_waitcnt(0);
                        if (lane == 0) st_flag(lb.flags + base + s, tag | kStatusAgg);
                        published = true;
                    }
                    if (++spins > lb.spin_limit) {
                        if (lane == 0) atomicOr(lb.error, 1u);
                        jstar = -1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                    continue;
                }
                if (first < 64) {
                    jstar = jhi - first;
                    break;
                }
                jhi -= 64;  // 64 aggregates in a row: keep looking further back
            }
        }
        if (lane == 0) s_jstar = jstar;
    }
    __syncthreads();

    // ---- fold: carry entering the segment for this wave's kSPW states
    const int64_t jstar = s_jstar;
    float c[kSPW];
#pragma unroll
    for (int q = 0; q < kSPW; ++q)
        c[q] = jstar >= 0 ? ld_coherent(lb.incl + (base + jstar) * (16 * 64) + (kSPW * wave + q) * 64 + lane) : 0.0f;
    for (int64_t j0 = jstar + 1; j0 < s; j0 += kFoldBatch) {
        float hb[kFoldBatch][kSPW], sb[kFoldBatch];
#pragma unroll
        for (int k = 0; k < kFoldBatch; ++k) {
            const int64_t j = j0 + k < s ? j0 + k : s - 1;
            const float* ag = lb.agg + (base + j) * (17 * 64);
            sb[k] = ld_coherent(ag + 16 * 64 + lane);
#pragma unroll
            for (int q = 0; q < kSPW; ++q) hb[k][q] = ld_coherent(ag + (kSPW * wave + q) * 64 + lane);
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
        float* ic = lb.incl + (base + s) * (16 * 64);
#pragma unroll
        for (int q = 0; q < kSPW; ++q) st_coherent(ic + (kSPW * wave + q) * 64 + lane, inc[q]);
        __builtin_amdgcn_s_waitcnt(0);
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
            v = fmaf(pw[q][w], v, hw);
        }
    }
    __syncthreads();
    if (s < S - 1 && threadIdx.x == 0) st_flag(lb.flags + base + s, tag | kStatusIncl);

    // ---- pass B: rerun the block from the state entering it; readout, skip, gate, store
#pragma unroll
    for (int n = 0; n < kMaxState; ++n) h[n] = s_h[wave][n][lane];

    // Recomputing the decays and writes is cheaper than holding pass A's 2 x 128 values per lane
    // across the look-back; the opaque copies of the step and rows (pin) also keep the compiler from
    // merging the two passes' identical expressions.
    float o8[8];
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
        const float uj = ur.get(j);
        float acc0 = skip * uj, acc1 = 0.0f;
        const float dtj = pin(dt[j]), dxj = pin(dtj * uj);
        float bv[kMaxState], cv[kMaxState];
        read_row(s_rows[wave][0][j], bv);
        read_row(s_rows[wave][1][j], cv);
#pragma unroll
        for (int n = 0; n < kMaxState; ++n) {
            const float yn = dtj * a2[n], an = exp2_hw(yn);
            if constexpr (ZOH) h[n] = fmaf(an, h[n], bv[n] * (zoh_gain(yn, an, dtj, ia[n]) * uj));
            else h[n] = fmaf(an, h[n], bv[n] * dxj);
            if (n & 1) acc1 = fmaf(cv[n], h[n], acc1);
            else acc0 = fmaf(cv[n], h[n], acc0);
        }
        float out = acc0 + acc1;
        if constexpr (GZ) out *= silu_f32(zr.get(j));
        o8[j % 8] = pin(out);
        if (j % 8 == 7 && active && p.out) store_chunk<IO, VEC>(static_cast<T*>(p.out) + row, tw + j - 7, L, o8);
        pin_states(h);
        __builtin_amdgcn_sched_barrier(0);
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
}

template <int W, typename IO, int NFIX, bool VEC, bool SP, bool GZ, bool ZOH, bool CK>
hipError_t launch_typed(const LbArgs& lb, hipStream_t s) {
    const int64_t blocks = lb.nbg * lb.S;
    hipLaunchKernelGGL((scan_fwd_kernel<W, IO, NFIX, VEC, SP, GZ, ZOH, CK>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(W * 64), 0, s, lb);
    return hipGetLastError();
}

// Zero-order hold, or the checkpointing pass of the backward (Euler only), or the plain forward.
template <int W, typename IO, int NFIX, bool VEC, bool SP, bool GZ>
hipError_t launch_zoh(const LbArgs& lb, hipStream_t s) {
    if (lb.a.zoh) return launch_typed<W, IO, NFIX, VEC, SP, GZ, true, false>(lb, s);
    if (lb.a.hblk) return launch_typed<W, IO, NFIX, VEC, SP, GZ, false, true>(lb, s);
    return launch_typed<W, IO, NFIX, VEC, SP, GZ, false, false>(lb, s);
}

template <int W, typename IO, int NFIX, bool VEC>
hipError_t launch_flags(const LbArgs& lb, hipStream_t s) {
    const bool sp = lb.a.softplus != 0, gz = lb.a.z != nullptr;
    if (sp) return gz ? launch_zoh<W, IO, NFIX, VEC, true, true>(lb, s) : launch_zoh<W, IO, NFIX, VEC, true, false>(lb, s);
    return gz ? launch_zoh<W, IO, NFIX, VEC, false, true>(lb, s) : launch_zoh<W, IO, NFIX, VEC, false, false>(lb, s);
}

template <int W, typename IO>
hipError_t launch_io(const LbArgs& lb, hipStream_t s) {
    const bool vec = lb.a.L % (16 / IO::bytes) == 0;
    if (lb.a.N == kMaxState)
        return vec ? launch_flags<W, IO, kMaxState, true>(lb, s) : launch_flags<W, IO, kMaxState, false>(lb, s);
    return vec ? launch_flags<W, IO, 0, true>(lb, s) : launch_flags<W, IO, 0, false>(lb, s);
}

int64_t segments(int64_t L, int seg) { return (L + seg - 1) / seg; }

}  // namespace

size_t scan_workspace_bytes(int64_t nb, int64_t nd, int64_t L) {
    const int64_t nbg = nb * ((nd + 63) / 64);
    const size_t slots = static_cast<size_t>(nbg * segments(L, kWavesPerGroup * kTok));
    const size_t flag_bytes = (slots * 4 + 255) & ~size_t(255);
    return kWorkspaceHeader + flag_bytes + slots * (17 + 16) * 64 * 4;
}

int64_t scan_max_blocks(int64_t nb, int64_t nd, int64_t L) {
    return nb * ((nd + 63) / 64) * segments(L, kWavesPerGroup * kTok);
}

int scan_segment_tokens(int64_t, int64_t, int64_t) { return kWavesPerGroup * kTok; }

int set_scan_wait_limit(int polls) { return g_spin_limit.exchange(polls > 0 ? polls : kSpinLimit); }

hipError_t launch_scan_fwd(const ScanArgs& a, bool io_bf16, void* workspace, uint32_t epoch, hipStream_t s) {
    constexpr int W = kWavesPerGroup;
    LbArgs lb;
    lb.a = a;
    lb.groups = (a.nd + 63) / 64;
    lb.nbg = a.nb * lb.groups;
    lb.S = segments(a.L, W * kTok);
    lb.epoch = epoch & 0x3fffffffu;
    char* ws = static_cast<char*>(workspace);
    const int64_t slots = lb.nbg * lb.S;  // at most the slots scan_workspace_bytes() provides for
    lb.error = reinterpret_cast<uint32_t*>(ws);
    lb.eager = lb.nbg < kEagerGroups ? 1u : 0u;
    lb.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    lb.flags = reinterpret_cast<uint32_t*>(ws + kWorkspaceHeader);
    const size_t flag_bytes = (static_cast<size_t>(slots) * 4 + 255) & ~size_t(255);
    lb.agg = reinterpret_cast<float*>(ws + kWorkspaceHeader + flag_bytes);
    lb.incl = lb.agg + slots * 17 * 64;
    return io_bf16 ? launch_io<W, bf16_io>(lb, s) : launch_io<W, f32_io>(lb, s);
}

}  // namespace ssm
