// scan_common.hpp - per-wave building blocks shared by the scan's forward and backward kernels
// (gfx950): a wave owns kTok consecutive tokens of 64 channels (lane = channel); these read and
// write its blocks of u, delta, z and out, keep u and z in the io format, stage the B and C rows of
// its tokens in LDS and read them back as broadcasts, and pin values to points of the program.
#pragma once

#include "ssm_device.hpp"

namespace ssm {
namespace scan {

constexpr int kTok = 16;  // tokens per wave

// kTok consecutive elements of one row starting at token t0 (zeros past the end); with VEC the
// row is read 8 tokens at a time in 16-byte vectors.
template <typename IO, bool VEC>
__device__ __forceinline__ void load_block(const typename IO::storage* __restrict__ row, int64_t t0, int64_t L,
                                           float (&v)[kTok]) {
    if (VEC && t0 + kTok <= L) {
#pragma unroll
        for (int c = 0; c < kTok; c += 8) {
            if constexpr (IO::bytes == 4) {
                const float4* q = reinterpret_cast<const float4*>(row + t0 + c);
                const float4 a = q[0], b = q[1];
                v[c] = a.x; v[c + 1] = a.y; v[c + 2] = a.z; v[c + 3] = a.w;
                v[c + 4] = b.x; v[c + 5] = b.y; v[c + 6] = b.z; v[c + 7] = b.w;
            } else {
                const uint4 q = *reinterpret_cast<const uint4*>(row + t0 + c);
                v[c] = bf16_lo(q.x); v[c + 1] = bf16_hi(q.x); v[c + 2] = bf16_lo(q.y); v[c + 3] = bf16_hi(q.y);
                v[c + 4] = bf16_lo(q.z); v[c + 5] = bf16_hi(q.z); v[c + 6] = bf16_lo(q.w); v[c + 7] = bf16_hi(q.w);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kTok; ++j) v[j] = (t0 + j < L) ? load_elem(row, t0 + j) : 0.0f;
    }
}

// Eight consecutive outputs of one row starting at token t0 (past the end: not stored); with VEC
// one or two 16-byte vector stores.
template <typename IO, bool VEC>
__device__ __forceinline__ void store_chunk(typename IO::storage* __restrict__ row, int64_t t0, int64_t L,
                                            const float (&v)[8]) {
    if (VEC && t0 + 8 <= L) {
        if constexpr (IO::bytes == 4) {
            float4* q = reinterpret_cast<float4*>(row + t0);
            q[0] = make_float4(v[0], v[1], v[2], v[3]);
            q[1] = make_float4(v[4], v[5], v[6], v[7]);
        } else {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[2 * k]));
                const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[2 * k + 1]));
                w[k] = lo | (hi << 16);
            }
            *reinterpret_cast<uint4*>(row + t0) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (t0 + j < L) store_elem(row, t0 + j, v[j]);
    }
}

// Four consecutive outputs of one row starting at token t0 (past the end: not stored); with VEC one
// 8-byte (bf16) or 16-byte (fp32) vector store.
template <typename IO, bool VEC>
__device__ __forceinline__ void store_chunk4(typename IO::storage* __restrict__ row, int64_t t0, int64_t L,
                                             const float (&v)[4]) {
    if (VEC && t0 + 4 <= L) {
        if constexpr (IO::bytes == 4) {
            *reinterpret_cast<float4*>(row + t0) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
            uint32_t w[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[2 * k]));
                const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[2 * k + 1]));
                w[k] = lo | (hi << 16);
            }
            *reinterpret_cast<uint2*>(row + t0) = make_uint2(w[0], w[1]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (t0 + j < L) store_elem(row, t0 + j, v[j]);
    }
}

// kTok values of one row held in registers in the io format: fp32 as is, bf16 two to a register
// (widened when read), so that u and z cost kTok/2 registers in bf16.
template <typename IO>
struct TokRow;
template <>
struct TokRow<f32_io> {
    float v[kTok];
    __device__ __forceinline__ float get(int j) const { return v[j]; }
};
template <>
struct TokRow<bf16_io> {
    uint32_t w[kTok / 2];
    __device__ __forceinline__ float get(int j) const { return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]); }
};

template <bool VEC>
__device__ __forceinline__ void load_tokrow(const float* __restrict__ row, int64_t t0, int64_t L, TokRow<f32_io>& r) {
    load_block<f32_io, VEC>(row, t0, L, r.v);
}
template <bool VEC>
__device__ __forceinline__ void load_tokrow(const uint16_t* __restrict__ row, int64_t t0, int64_t L, TokRow<bf16_io>& r) {
    if (VEC && t0 + kTok <= L) {
#pragma unroll
        for (int c = 0; c < kTok; c += 8) {
            const uint4 q = *reinterpret_cast<const uint4*>(row + t0 + c);
            r.w[c / 2] = q.x; r.w[c / 2 + 1] = q.y; r.w[c / 2 + 2] = q.z; r.w[c / 2 + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < kTok / 2; ++k) {
            const uint32_t lo = t0 + 2 * k < L ? row[t0 + 2 * k] : 0u;
            const uint32_t hi = t0 + 2 * k + 1 < L ? row[t0 + 2 * k + 1] : 0u;
            r.w[k] = lo | (hi << 16);
        }
    }
}

// An opaque copy: chains a value to this point of the program, so that work derived from it is not
// computed early and held in registers.
__device__ __forceinline__ float pin(float v) {
    asm("" : "+v"(v));
    return v;
}

// Opaque copies of the 16 states: the end of one token's work, which the next token's must follow.
__device__ __forceinline__ void pin_states(float (&h)[kMaxState]) {
    asm("" : "+v"(h[0]), "+v"(h[1]), "+v"(h[2]), "+v"(h[3]), "+v"(h[4]), "+v"(h[5]), "+v"(h[6]), "+v"(h[7]),
             "+v"(h[8]), "+v"(h[9]), "+v"(h[10]), "+v"(h[11]), "+v"(h[12]), "+v"(h[13]), "+v"(h[14]), "+v"(h[15]));
}

// Stage the B (or C) rows of one wave's kTok tokens into LDS as fp32: rows[j][n] = row t0 + j,
// state n (0 past the end of the sequence and for n >= N). The block of kTok rows is contiguous in
// memory when N = 16, so each lane loads kE consecutive elements with one vector load.
template <typename IO, int NFIX>
__device__ __forceinline__ void stage_rows(const typename IO::storage* __restrict__ base, int64_t t0, int64_t L, int N,
                                           int lane, float (*rows)[kMaxState]) {
    constexpr int kE = kTok * kMaxState / 64;  // elements per lane: 2 or 4
    static_assert(kE == 2 || kE == 4, "row staging assumes 8 or 16 tokens per wave");
    const int i = kE * lane;  // elements i .. i + kE - 1 of the kTok x 16 block, all in row i / 16
    float v[kE];
    if (NFIX == kMaxState && t0 + kTok <= L) {
        if constexpr (IO::bytes == 4) {
            if constexpr (kE == 2) {
                const float2 q = *reinterpret_cast<const float2*>(base + t0 * kMaxState + i);
                v[0] = q.x; v[1] = q.y;
            } else {
                const float4 q = *reinterpret_cast<const float4*>(base + t0 * kMaxState + i);
                v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
            }
        } else {
            if constexpr (kE == 2) {
                const uint32_t q = *reinterpret_cast<const uint32_t*>(base + t0 * kMaxState + i);
                v[0] = bf16_lo(q); v[1] = bf16_hi(q);
            } else {
                const uint2 q = *reinterpret_cast<const uint2*>(base + t0 * kMaxState + i);
                v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
            }
        }
    } else {
        const int j = i / kMaxState, n = i % kMaxState;  // n + kE <= 16
        const bool in = t0 + j < L;
#pragma unroll
        for (int e = 0; e < kE; ++e) v[e] = in && n + e < N ? load_elem(base, (t0 + j) * N + n + e) : 0.0f;
    }
    float* dst = &rows[i / kMaxState][i % kMaxState];
    if constexpr (kE == 2) *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
    else *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
}

// One lane's share of a wave's kTok x 16 block of B (or C) rows, as the raw words loaded from memory
// (N = 16 and the whole block inside the sequence: the block is contiguous). Split from the widening
// into LDS (put_rows) so that the load is in flight together with the segment's other loads: the
// compiler waits for a loaded value at its first use, so a load whose value is used right away costs a
// whole memory round trip before the next load is even issued.
template <typename IO>
struct RowWords {
    static constexpr int kE = kTok * kMaxState / 64;  // elements per lane
    uint32_t w[kE * IO::bytes / 4];
};

template <typename IO>
__device__ __forceinline__ void fetch_rows(const typename IO::storage* __restrict__ base, int64_t t0, int lane,
                                           RowWords<IO>& r) {
    constexpr int kE = RowWords<IO>::kE;
    static_assert(kE == 4, "row fetch assumes 16 tokens per wave");
    const typename IO::storage* q = base + t0 * kMaxState + kE * lane;
    if constexpr (IO::bytes == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(q);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(q);
        r.w[0] = v.x; r.w[1] = v.y;
    }
}

// The fetched words widened to fp32 into rows[j][n] (the layout stage_rows writes).
template <typename IO>
__device__ __forceinline__ void put_rows(const RowWords<IO>& r, int lane, float (*rows)[kMaxState]) {
    constexpr int kE = RowWords<IO>::kE;
    float v[kE];
    if constexpr (IO::bytes == 4) {
#pragma unroll
        for (int e = 0; e < kE; ++e) v[e] = __uint_as_float(r.w[e]);
    } else {
        v[0] = bf16_lo(r.w[0]); v[1] = bf16_hi(r.w[0]); v[2] = bf16_lo(r.w[1]); v[3] = bf16_hi(r.w[1]);
    }
    const int i = kE * lane;
    *reinterpret_cast<float4*>(&rows[i / kMaxState][i % kMaxState]) = make_float4(v[0], v[1], v[2], v[3]);
}

// Four consecutive states (4k .. 4k + 3) of one token's row from LDS: an LDS broadcast, like read_row.
__device__ __forceinline__ float4 read_quad(const float* row, int k) {
    return reinterpret_cast<const float4*>(row)[k];
}

// One token's 16-element row from LDS. Every lane reads the same address: an LDS broadcast, so the
// values arrive in ordinary VGPRs and the arithmetic that uses them needs no cross-lane operand.
__device__ __forceinline__ void read_row(const float* row, float (&v)[kMaxState]) {
    const float4* q = reinterpret_cast<const float4*>(row);
#pragma unroll
    for (int k = 0; k < kMaxState / 4; ++k) {
        const float4 x = q[k];
        v[4 * k] = x.x;
        v[4 * k + 1] = x.y;
        v[4 * k + 2] = x.z;
        v[4 * k + 3] = x.w;
    }
}

}  // namespace scan
}  // namespace ssm
