// abi.cpp - the extern "C" boundary of libssmscan.so (declared in include/ssm_scan.h).
//
// Every argument is checked here before any HIP call; a rejected call launches nothing, returns
// its status and leaves a message in thread-local storage. Valid calls enqueue the kernels on the
// caller's stream and return without synchronising.
#include "ssm_scan.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "ssm_kernels.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return SSM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b without overflow past limit; false if it would exceed it.
bool mul_le(int64_t a, int64_t b, int64_t limit, int64_t* r) {
    if (a > 0 && b > limit / a) return false;
    *r = a * b;
    return true;
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    if (!a || !b) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

constexpr int64_t kMaxElems = int64_t(1) << 46;       // per tensor; far beyond any device memory
constexpr int64_t kMaxBlocks = (int64_t(1) << 31) - 1;  // grid x limit with 64-lane workgroups

int check_dtype(int io_dtype) {
    if (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16)
        return fail(SSM_ERR_BAD_DTYPE, "io_dtype %d is not SSM_DTYPE_F32 (0) or SSM_DTYPE_BF16 (1)", io_dtype);
    return SSM_OK;
}

int check_flags(unsigned flags, const char* fn) {
    if (flags & ~static_cast<unsigned>(SSM_FLAG_ZOH))
        return fail(SSM_ERR_BAD_FLAGS, "%s: unknown flag bits 0x%x", fn, flags & ~static_cast<unsigned>(SSM_FLAG_ZOH));
    return SSM_OK;
}

#define CHECK_NONNULL(p) \
    if (!(p)) return fail(SSM_ERR_NULL_POINTER, "%s: required pointer '" #p "' is NULL", fn)
#define CHECK_ALIGN(p) \
    if ((p) && !aligned16(p)) return fail(SSM_ERR_MISALIGNED, "%s: pointer '" #p "' (%p) is not 16-byte aligned", fn, (const void*)(p))

}  // namespace

extern "C" {

int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* delta_bias, int softplus_flag,
                 void* out, float* last_state, int64_t batch, int64_t dim, int64_t seqlen,
                 int64_t dstate, int io_dtype, void* stream) {
    return ssm_scan_fwd_ex(u, delta, A, B, C, D, z, delta_bias, softplus_flag, out, last_state, batch, dim, seqlen,
                           dstate, io_dtype, 0u, stream);
}

int ssm_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B, const void* C,
                    const float* D, const void* z, const float* delta_bias, int softplus_flag,
                    void* out, float* last_state, int64_t batch, int64_t dim, int64_t seqlen,
                    int64_t dstate, int io_dtype, unsigned flags, void* stream) {
    const char* fn = "ssm_scan_fwd";
    if (int s = check_dtype(io_dtype)) return s;
    if (int s = check_flags(flags, fn)) return s;
    CHECK_NONNULL(u);
    CHECK_NONNULL(delta);
    CHECK_NONNULL(A);
    CHECK_NONNULL(B);
    CHECK_NONNULL(C);
    CHECK_NONNULL(out);
    if (batch < 1 || dim < 1 || seqlen < 1)
        return fail(SSM_ERR_BAD_SHAPE, "%s: batch=%lld dim=%lld seqlen=%lld must all be >= 1", fn,
                    (long long)batch, (long long)dim, (long long)seqlen);
    if (dstate < 1 || dstate > SSM_MAX_DSTATE)
        return fail(SSM_ERR_BAD_SHAPE, "%s: dstate=%lld must be in [1, %d]", fn, (long long)dstate, SSM_MAX_DSTATE);
    int64_t rows, elems, bs, bc, blocks;
    if (!mul_le(batch, dim, kMaxElems, &rows) || !mul_le(rows, seqlen, kMaxElems, &elems) ||
        !mul_le(batch, seqlen, kMaxElems, &bs) || !mul_le(bs, dstate, kMaxElems, &bc) ||
        !mul_le((dim + 63) / 64, batch, kMaxBlocks, &blocks))
        return fail(SSM_ERR_BAD_SHAPE, "%s: sizes batch=%lld dim=%lld seqlen=%lld are too large", fn,
                    (long long)batch, (long long)dim, (long long)seqlen);
    CHECK_ALIGN(u);
    CHECK_ALIGN(delta);
    CHECK_ALIGN(A);
    CHECK_ALIGN(B);
    CHECK_ALIGN(C);
    CHECK_ALIGN(D);
    CHECK_ALIGN(z);
    CHECK_ALIGN(delta_bias);
    CHECK_ALIGN(out);
    CHECK_ALIGN(last_state);
    const int64_t es = io_dtype == SSM_DTYPE_F32 ? 4 : 2;
    const int64_t io_bytes = elems * es;
    if (overlaps(out, io_bytes, u, io_bytes) || overlaps(out, io_bytes, delta, io_bytes) ||
        overlaps(out, io_bytes, z, io_bytes) || overlaps(out, io_bytes, B, bc * es) ||
        overlaps(out, io_bytes, C, bc * es))
        return fail(SSM_ERR_BAD_SHAPE, "%s: out overlaps an input tensor", fn);
    if (overlaps(last_state, rows * dstate * 4, out, io_bytes) || overlaps(last_state, rows * dstate * 4, u, io_bytes) ||
        overlaps(last_state, rows * dstate * 4, delta, io_bytes))
        return fail(SSM_ERR_BAD_SHAPE, "%s: last_state overlaps another tensor", fn);

    if (ssm::scan_max_blocks(batch, dim, seqlen) > kMaxBlocks)
        return fail(SSM_ERR_BAD_SHAPE, "%s: batch=%lld dim=%lld seqlen=%lld need too many workgroups", fn,
                    (long long)batch, (long long)dim, (long long)seqlen);

    ssm::ScanArgs a{u, delta, A, B, C, D, z, delta_bias, out, last_state, batch, dim, seqlen,
                    static_cast<int>(dstate), softplus_flag != 0, (flags & SSM_FLAG_ZOH) != 0};
    const bool bf16 = io_dtype == SSM_DTYPE_BF16;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const hipError_t e = ssm::with_scan_workspace(
        hs, ssm::scan_workspace_bytes(batch, dim, seqlen),
        [&](void* ws, uint32_t epoch) { return ssm::launch_scan_fwd(a, bf16, ws, epoch, hs); });
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    return ok();
}

int ssm_state_update(float* state, const void* x, const void* delta, const float* A, const void* B,
                     const void* C, const float* D, const void* z, void* out, int64_t batch,
                     int64_t dim, int64_t dstate, int io_dtype, void* stream) {
    return ssm_state_update_ex(state, x, delta, A, B, C, D, z, out, batch, dim, dstate, io_dtype, 0u, stream);
}

int ssm_state_update_ex(float* state, const void* x, const void* delta, const float* A, const void* B,
                     const void* C, const float* D, const void* z, void* out, int64_t batch,
                     int64_t dim, int64_t dstate, int io_dtype, unsigned flags, void* stream) {
    const char* fn = "ssm_state_update";
    if (int s = check_dtype(io_dtype)) return s;
    if (int s = check_flags(flags, fn)) return s;
    CHECK_NONNULL(state);
    CHECK_NONNULL(x);
    CHECK_NONNULL(delta);
    CHECK_NONNULL(A);
    CHECK_NONNULL(B);
    CHECK_NONNULL(C);
    CHECK_NONNULL(out);
    if (batch < 1 || dim < 1)
        return fail(SSM_ERR_BAD_SHAPE, "%s: batch=%lld dim=%lld must be >= 1", fn, (long long)batch, (long long)dim);
    if (dstate < 1 || dstate > SSM_MAX_DSTATE)
        return fail(SSM_ERR_BAD_SHAPE, "%s: dstate=%lld must be in [1, %d]", fn, (long long)dstate, SSM_MAX_DSTATE);
    int64_t rows, blocks;
    if (!mul_le(batch, dim, kMaxElems, &rows) || !mul_le((dim + 63) / 64, batch, kMaxBlocks, &blocks))
        return fail(SSM_ERR_BAD_SHAPE, "%s: sizes batch=%lld dim=%lld are too large", fn, (long long)batch, (long long)dim);
    CHECK_ALIGN(state);
    CHECK_ALIGN(x);
    CHECK_ALIGN(delta);
    CHECK_ALIGN(A);
    CHECK_ALIGN(B);
    CHECK_ALIGN(C);
    CHECK_ALIGN(D);
    CHECK_ALIGN(z);
    CHECK_ALIGN(out);
    const int64_t es = io_dtype == SSM_DTYPE_F32 ? 4 : 2;
    const int64_t sbytes = rows * dstate * 4;
    if (overlaps(out, rows * es, state, sbytes) || overlaps(out, rows * es, x, rows * es) ||
        overlaps(out, rows * es, delta, rows * es) || overlaps(out, rows * es, z, rows * es) ||
        overlaps(state, sbytes, x, rows * es) || overlaps(state, sbytes, delta, rows * es) ||
        overlaps(state, sbytes, z, rows * es))
        return fail(SSM_ERR_BAD_SHAPE, "%s: out or state overlaps another tensor", fn);

    ssm::UpdateArgs a{state, x, delta, A, B, C, D, z, out, batch, dim, static_cast<int>(dstate),
                      (flags & SSM_FLAG_ZOH) != 0};
    const hipError_t e = ssm::launch_state_update(a, io_dtype == SSM_DTYPE_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

int ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* delta_bias, int softplus_flag, const void* dout, void* du, void* ddelta,
                 float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias, int64_t batch,
                 int64_t dim, int64_t seqlen, int64_t dstate, int io_dtype, void* stream) {
    const char* fn = "ssm_scan_bwd";
    if (int s = check_dtype(io_dtype)) return s;
    CHECK_NONNULL(u);
    CHECK_NONNULL(delta);
    CHECK_NONNULL(A);
    CHECK_NONNULL(B);
    CHECK_NONNULL(C);
    CHECK_NONNULL(dout);
    CHECK_NONNULL(du);
    CHECK_NONNULL(ddelta);
    CHECK_NONNULL(dA);
    CHECK_NONNULL(dB);
    CHECK_NONNULL(dC);
    if (z && !dz) return fail(SSM_ERR_NULL_POINTER, "%s: dz is required when z is given", fn);
    if (batch < 1 || dim < 1 || seqlen < 1)
        return fail(SSM_ERR_BAD_SHAPE, "%s: batch=%lld dim=%lld seqlen=%lld must be >= 1", fn, (long long)batch,
                    (long long)dim, (long long)seqlen);
    if (dstate < 1 || dstate > SSM_MAX_DSTATE)
        return fail(SSM_ERR_BAD_SHAPE, "%s: dstate=%lld must be in [1, %d]", fn, (long long)dstate, SSM_MAX_DSTATE);
    int64_t rows, elems, bc;
    if (!mul_le(batch, dim, kMaxElems, &rows) || !mul_le(rows, seqlen, kMaxElems, &elems) ||
        !mul_le(batch * seqlen, dstate, kMaxElems, &bc) || ssm::scan_max_blocks(batch, dim, seqlen) > kMaxBlocks)
        return fail(SSM_ERR_BAD_SHAPE, "%s: sizes batch=%lld dim=%lld seqlen=%lld are too large", fn,
                    (long long)batch, (long long)dim, (long long)seqlen);
    CHECK_ALIGN(u);
    CHECK_ALIGN(delta);
    CHECK_ALIGN(A);
    CHECK_ALIGN(B);
    CHECK_ALIGN(C);
    CHECK_ALIGN(D);
    CHECK_ALIGN(z);
    CHECK_ALIGN(delta_bias);
    CHECK_ALIGN(dout);
    CHECK_ALIGN(du);
    CHECK_ALIGN(ddelta);
    CHECK_ALIGN(dA);
    CHECK_ALIGN(dB);
    CHECK_ALIGN(dC);
    CHECK_ALIGN(dD);
    CHECK_ALIGN(dz);
    CHECK_ALIGN(ddelta_bias);
    const int64_t es = io_dtype == SSM_DTYPE_F32 ? 4 : 2;
    const int64_t ib = elems * es;
    const void* ins[] = {u, delta, dout, z};
    void* outs[] = {du, ddelta, dz};
    for (void* o : outs)
        for (const void* in : ins)
            if (o && in && overlaps(o, ib, in, ib)) return fail(SSM_ERR_BAD_SHAPE, "%s: a gradient overlaps an input", fn);
    if (overlaps(dB, bc * 4, dC, bc * 4) || overlaps(du, ib, ddelta, ib))
        return fail(SSM_ERR_BAD_SHAPE, "%s: gradient outputs overlap", fn);

    ssm::BwdArgs q{};
    q.a = ssm::ScanArgs{u, delta, A, B, C, D, z, delta_bias, nullptr, nullptr, batch, dim, seqlen,
                        static_cast<int>(dstate), softplus_flag != 0, 0};
    q.dout = dout;
    q.du = du;
    q.ddelta = ddelta;
    q.dz = dz;
    q.dA = dA;
    q.dB = dB;
    q.dC = dC;
    q.dD = dD;
    q.dbias = ddelta_bias;
    const bool bf16 = io_dtype == SSM_DTYPE_BF16;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const size_t scan_bytes = ssm::scan_workspace_bytes(batch, dim, seqlen);
    const hipError_t e = ssm::with_scan_workspace(
        hs, scan_bytes + ssm::scan_bwd_extra_bytes(batch, dim, seqlen), [&](void* ws, uint32_t epoch) {
            return ssm::launch_scan_bwd(q, bf16, ws, epoch, static_cast<char*>(ws) + scan_bytes, hs);
        });
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    return ok();
}

int ssm_causal_conv1d(const void* x, const float* weight, const float* bias, int silu_flag, void* out,
                      int64_t batch, int64_t dim, int64_t seqlen, int64_t width, int io_dtype, void* stream) {
    const char* fn = "ssm_causal_conv1d";
    if (int s = check_dtype(io_dtype)) return s;
    CHECK_NONNULL(x);
    CHECK_NONNULL(weight);
    CHECK_NONNULL(out);
    if (batch < 1 || dim < 1 || seqlen < 1)
        return fail(SSM_ERR_BAD_SHAPE, "%s: batch=%lld dim=%lld seqlen=%lld must be >= 1", fn, (long long)batch,
                    (long long)dim, (long long)seqlen);
    if (width < 1 || width > SSM_MAX_CONV_WIDTH)
        return fail(SSM_ERR_BAD_SHAPE, "%s: width=%lld must be in [1, %d]", fn, (long long)width, SSM_MAX_CONV_WIDTH);
    int64_t rows, elems;
    if (!mul_le(batch, dim, kMaxElems, &rows) || !mul_le(rows, seqlen, kMaxElems, &elems) ||
        ssm::conv_max_blocks(batch, dim, seqlen) > kMaxBlocks)
        return fail(SSM_ERR_BAD_SHAPE, "%s: sizes batch=%lld dim=%lld seqlen=%lld are too large", fn,
                    (long long)batch, (long long)dim, (long long)seqlen);
    CHECK_ALIGN(x);
    CHECK_ALIGN(weight);
    CHECK_ALIGN(bias);
    CHECK_ALIGN(out);
    const int64_t es = io_dtype == SSM_DTYPE_F32 ? 4 : 2;
    if (overlaps(out, elems * es, x, elems * es))
        return fail(SSM_ERR_BAD_SHAPE, "%s: out overlaps x", fn);
    ssm::ConvArgs a{x, weight, bias, out, nullptr, batch, dim, seqlen, static_cast<int>(width), silu_flag != 0};
    const hipError_t e = ssm::launch_causal_conv1d(a, io_dtype == SSM_DTYPE_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

int ssm_conv_window_update(float* window, const void* x, const float* weight, const float* bias, int silu_flag,
                           void* out, int64_t batch, int64_t dim, int64_t width, int io_dtype, void* stream) {
    const char* fn = "ssm_conv_window_update";
    if (int s = check_dtype(io_dtype)) return s;
    CHECK_NONNULL(window);
    CHECK_NONNULL(x);
    CHECK_NONNULL(weight);
    CHECK_NONNULL(out);
    if (batch < 1 || dim < 1)
        return fail(SSM_ERR_BAD_SHAPE, "%s: batch=%lld dim=%lld must be >= 1", fn, (long long)batch, (long long)dim);
    if (width < 1 || width > SSM_MAX_CONV_WIDTH)
        return fail(SSM_ERR_BAD_SHAPE, "%s: width=%lld must be in [1, %d]", fn, (long long)width, SSM_MAX_CONV_WIDTH);
    int64_t rows, wbytes;
    if (!mul_le(batch, dim, kMaxElems, &rows) || !mul_le(rows, width * 4, kMaxElems, &wbytes) ||
        (rows + 255) / 256 > kMaxBlocks)
        return fail(SSM_ERR_BAD_SHAPE, "%s: sizes batch=%lld dim=%lld are too large", fn, (long long)batch,
                    (long long)dim);
    CHECK_ALIGN(window);
    CHECK_ALIGN(x);
    CHECK_ALIGN(weight);
    CHECK_ALIGN(bias);
    CHECK_ALIGN(out);
    const int64_t es = io_dtype == SSM_DTYPE_F32 ? 4 : 2;
    if (overlaps(out, rows * es, x, rows * es) || overlaps(out, rows * es, window, wbytes) ||
        overlaps(window, wbytes, x, rows * es))
        return fail(SSM_ERR_BAD_SHAPE, "%s: out, window or x overlap", fn);
    ssm::ConvArgs a{x, weight, bias, out, window, batch, dim, 1, static_cast<int>(width), silu_flag != 0};
    const hipError_t e = ssm::launch_conv_window_update(a, io_dtype == SSM_DTYPE_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

int ssm_stream_check(void* stream) {
    uint32_t flags = 0;
    const hipError_t e = ssm::take_workspace_errors(static_cast<hipStream_t>(stream), &flags);
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "ssm_stream_check: %s", hipGetErrorString(e));
    if (flags)
        return fail(SSM_ERR_DEVICE_WAIT, "ssm_stream_check: a scan on this stream timed out waiting for another "
                                         "workgroup (flags 0x%x); its outputs are not valid", flags);
    return ok();
}

int ssm_release_workspaces(void) {
    const hipError_t e = ssm::release_workspaces();
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "ssm_release_workspaces: %s", hipGetErrorString(e));
    return ok();
}

const char* ssm_status_string(int status) {
    switch (status) {
        case SSM_OK: return "SSM_OK";
        case SSM_ERR_NULL_POINTER: return "SSM_ERR_NULL_POINTER";
        case SSM_ERR_BAD_SHAPE: return "SSM_ERR_BAD_SHAPE";
        case SSM_ERR_BAD_DTYPE: return "SSM_ERR_BAD_DTYPE";
        case SSM_ERR_MISALIGNED: return "SSM_ERR_MISALIGNED";
        case SSM_ERR_HIP: return "SSM_ERR_HIP";
        case SSM_ERR_DEVICE_WAIT: return "SSM_ERR_DEVICE_WAIT";
        case SSM_ERR_BAD_FLAGS: return "SSM_ERR_BAD_FLAGS";
        default: return "SSM_ERR_UNKNOWN";
    }
}

const char* ssm_last_error_message(void) { return g_last_error; }

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

int ssm_set_wait_limit(int polls) { return ssm::set_scan_wait_limit(polls); }

int ssm_scan_segment_tokens(int64_t batch, int64_t dim, int64_t seqlen) {
    if (batch < 1 || dim < 1 || seqlen < 1) return 0;
    return ssm::scan_segment_tokens(batch, dim, seqlen);
}

}  // extern "C"
