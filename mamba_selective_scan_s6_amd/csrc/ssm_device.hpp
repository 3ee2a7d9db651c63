// ssm_device.hpp - device-side helpers shared by the selective-scan kernels (gfx950).
//
// Element types: io tensors are fp32 or bf16 (carried as uint16 bit patterns); every value is
// widened to fp32 on load and all arithmetic is fp32. bf16 results are rounded to nearest even
// by the hardware conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr int kMaxState = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct f32_io {
    using storage = float;
    static constexpr int bytes = 4;
};
struct bf16_io {
    using storage = uint16_t;
    static constexpr int bytes = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

__device__ __forceinline__ void store_elem(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, int64_t i, float v) {
    __bf16 h = static_cast<__bf16>(v);  // v_cvt_pk_bf16_f32: round to nearest even
    p[i] = __builtin_bit_cast(uint16_t, h);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit (v_log_f32).
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// log(1 + e) for e in [0, 1]. Below 1/16 a 6-term Taylor series (truncation < e^6/7, i.e.
// < 1e-8 relative); above, log2(1 + e) * ln 2 where 1 + e >= 1.0625 keeps the hardware log's
// error small relative to the result.
__device__ __forceinline__ float log1p_unit(float e) {
    float s = fmaf(e, -1.0f / 6.0f, 1.0f / 5.0f);
    s = fmaf(e, s, -0.25f);
    s = fmaf(e, s, 1.0f / 3.0f);
    s = fmaf(e, s, -0.5f);
    s = fmaf(e, s, 1.0f);
    const float series = e * s;
    const float direct = log2_hw(1.0f + e) * kLn2;
    return e < 0.0625f ? series : direct;
}

// softplus(r) = log(1 + e^r) = max(r, 0) + log1p(e^{-|r|}).
__device__ __forceinline__ float softplus_f32(float r) {
    const float e = exp2_hw(-fabsf(r) * kLog2e);
    return fmaxf(r, 0.0f) + log1p_unit(e);
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^{-z}); e^{-z} overflowing to inf gives -0.
__device__ __forceinline__ float silu_f32(float z) {
    const float e = exp2_hw(-z * kLog2e);
    return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// Exact zero-order-hold input gain (e^{Delta a} - 1) / a for one (step, state) ("Module 19", The
// Math: the discretised input matrix; it tends to Delta as Delta a -> 0), given y = Delta a log2(e)
// and abar = 2^y. Below |Delta a| = 1/8 it is Delta (e^x - 1)/x from a 5-term series in x = Delta a
// (truncation < x^5/720 < 5e-8 relative), where abar - 1 would lose digits to cancellation; above,
// (abar - 1) / a, whose relative error stays below ~1e-6 because |abar - 1| > 0.117 there.
constexpr float kZohSmallY = 0.125f / kLn2;  // |y| below which the series is used
__device__ __forceinline__ float zoh_gain(float y, float abar, float dt, float inv_a) {
    constexpr float c1 = kLn2 / 2.0f, c2 = kLn2 * kLn2 / 6.0f, c3 = kLn2 * kLn2 * kLn2 / 24.0f,
                    c4 = kLn2 * kLn2 * kLn2 * kLn2 / 120.0f;
    const float phi = fmaf(y, fmaf(y, fmaf(y, fmaf(y, c4, c3), c2), c1), 1.0f);  // (e^x - 1)/x, x = y ln 2
    return fabsf(y) < kZohSmallY ? dt * phi : (abar - 1.0f) * inv_a;
}

}  // namespace ssm
