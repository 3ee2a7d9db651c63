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
#include <initializer_list>

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

// True if the range [w, w + wbytes) that a call writes overlaps any of the other (non-NULL) tensors.
bool overlaps_any(const void* w, int64_t wbytes, std::initializer_list<const void*> tensors,
                  std::initializer_list<int64_t> sizes) {
    auto sz = sizes.begin();
    for (const void* t : tensors) {
        if (t && overlaps(w, wbytes, t, *sz)) return true;
        ++sz;
    }
    return false;
}

constexpr int64_t kMaxElems = int64_t(1) << 46;       // per tensor; far beyond any device memory
constexpr int64_t kMaxBlocks = (int64_t(1) << 31) - 1;  // grid x limit with 64-lane workgroups
constexpr int64_t kSsdMaxSeqlen = int64_t(1) << 35;      // ssm_ssd_scan: a workgroup counts its chunks in 32 bits
constexpr int64_t kSsdMaxRow = int64_t(1) << 24;         // ssm_ssd_scan: elements per token of x and of b, c

int check_dtype(int io_dtype) {
    if (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16)
        return fail(SSM_ERR_BAD_DTYPE, "io_dtype %d is not SSM_DTYPE_F32 (0) or SSM_DTYPE_BF16 (1)", io_dtype);
    return SSM_OK;
}

int check_flags(unsigned flags, const char* fn) {
    constexpr unsigned known = SSM_FLAG_ZOH | SSM_FLAG_OUT_F32;
    if (flags & ~known) return fail(SSM_ERR_BAD_FLAGS, "%s: unknown flag bits 0x%x", fn, flags & ~known);
    return SSM_OK;
}

// The scan part of a backward workspace, rounded up so that the backward's own buffers after it stay
// 256-byte aligned.
size_t bwd_scan_part(size_t bytes) { return (bytes + 255) & ~size_t(255); }

// A caller's workspace: present, 16-byte aligned, large enough, and not overlapping any tensor.
int check_workspace(const char* fn, const void* ws, size_t have, size_t need,
                    std::initializer_list<const void*> tensors, std::initializer_list<int64_t> sizes) {
    if (!ws) return fail(SSM_ERR_WORKSPACE, "%s: workspace is NULL (see the _workspace_size query)", fn);
    if (!aligned16(ws)) return fail(SSM_ERR_MISALIGNED, "%s: workspace (%p) is not 16-byte aligned", fn, ws);
    if (have < need)
        return fail(SSM_ERR_WORKSPACE, "%s: workspace has %zu bytes, this call needs %zu", fn, have, need);
    auto sz = sizes.begin();
    for (const void* t : tensors) {
        if (t && overlaps(ws, static_cast<int64_t>(need), t, *sz))
            return fail(SSM_ERR_WORKSPACE, "%s: workspace overlaps a tensor argument", fn);
        ++sz;
    }
    return SSM_OK;
}

#define CHECK_NONNULL(p) \
    if (!(p)) return fail(SSM_ERR_NULL_POINTER, "%s: required pointer '" #p "' is NULL", fn)
#define CHECK_ALIGN(p) \
    if ((p) && !aligned16(p)) return fail(SSM_ERR_MISALIGNED, "%s: pointer '" #p "' (%p) is not 16-byte aligned", fn, (const void*)(p))

}  // namespace

extern "C" {

size_t ssm_scan_fwd_workspace_size(int64_t batch, int64_t dim, int64_t seqlen) {
    if (batch < 1 || dim < 1 || seqlen < 1) return 0;
    int64_t blocks;
    if (!mul_le(ssm::ceil_div(dim, 64), batch, kMaxBlocks, &blocks) || ssm::scan_max_blocks(batch, dim, seqlen) > kMaxBlocks)
        return 0;
    return ssm::scan_workspace_bytes(batch, dim, seqlen);
}

int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* delta_bias, int softplus_flag,
                 void* out, float* last_state, int64_t batch, int64_t dim, int64_t seqlen,
                 int64_t dstate, int io_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return ssm_scan_fwd_ex(u, delta, A, B, C, D, z, delta_bias, softplus_flag, out, last_state, batch, dim, seqlen,
                           dstate, io_dtype, 0u, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The forward scan behind both entry points: the caller's workspace, or (noalloc) the library's device
// array, which is looked up after every other check has passed.
int scan_fwd_impl(const char* fn, const void* u, const void* delta, const float* A, const void* B, const void* C,
                  const float* D, const void* z, const float* delta_bias, int softplus_flag, void* out,
                  float* last_state, int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int io_dtype,
                  unsigned flags, void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
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
        !mul_le(ssm::ceil_div(dim, 64), batch, kMaxBlocks, &blocks))
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
    const int64_t out_bytes = elems * ((flags & SSM_FLAG_OUT_F32) ? 4 : es);
    const int64_t sbytes = rows * dstate * 4, abytes = dim * dstate * 4, cbytes = dim * 4;
    if (overlaps_any(out, out_bytes, {u, delta, z, B, C, A, D, delta_bias, last_state},
                     {io_bytes, io_bytes, io_bytes, bc * es, bc * es, abytes, cbytes, cbytes, sbytes}))
        return fail(SSM_ERR_BAD_SHAPE, "%s: out overlaps another tensor argument", fn);
    if (last_state && overlaps_any(last_state, sbytes, {u, delta, z, B, C, A, D, delta_bias},
                                   {io_bytes, io_bytes, io_bytes, bc * es, bc * es, abytes, cbytes, cbytes}))
        return fail(SSM_ERR_BAD_SHAPE, "%s: last_state overlaps another tensor argument", fn);

    if (ssm::scan_max_blocks(batch, dim, seqlen) > kMaxBlocks)
        return fail(SSM_ERR_BAD_SHAPE, "%s: batch=%lld dim=%lld seqlen=%lld need too many workgroups", fn,
                    (long long)batch, (long long)dim, (long long)seqlen);

    const size_t need = ssm::scan_workspace_bytes(batch, dim, seqlen);
    if (noalloc) {
        if (need > ssm::kNoAllocScratchBytes)
            return fail(SSM_ERR_WORKSPACE, "%s: batch=%lld dim=%lld seqlen=%lld need %zu bytes of workspace, more than "
                        "the %zu this entry point holds; use ssm_scan_fwd with a workspace", fn, (long long)batch,
                        (long long)dim, (long long)seqlen, need, ssm::kNoAllocScratchBytes);
        const hipError_t e = ssm::noalloc_workspace(static_cast<hipStream_t>(stream), &workspace);
        if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    } else if (int st = check_workspace(fn, workspace, workspace_bytes, need,
                                        {u, delta, z, B, C, out, last_state, A, D, delta_bias},
                                        {io_bytes, io_bytes, io_bytes, bc * es, bc * es, out_bytes, rows * dstate * 4,
                                         dim * dstate * 4, dim * 4, dim * 4})) {
        return st;
    }

    ssm::ScanArgs a{u, delta, A, B, C, D, z, delta_bias, out, last_state, batch, dim, seqlen,
                    static_cast<int>(dstate), softplus_flag != 0, (flags & SSM_FLAG_ZOH) != 0};
    a.out_f32 = (flags & SSM_FLAG_OUT_F32) != 0;
    const hipError_t e = ssm::launch_scan_fwd(a, io_dtype == SSM_DTYPE_BF16, workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int ssm_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B, const void* C,
                    const float* D, const void* z, const float* delta_bias, int softplus_flag,
                    void* out, float* last_state, int64_t batch, int64_t dim, int64_t seqlen,
                    int64_t dstate, int io_dtype, unsigned flags, void* workspace, size_t workspace_bytes,
                    void* stream) {
    return scan_fwd_impl("ssm_scan_fwd", u, delta, A, B, C, D, z, delta_bias, softplus_flag, out, last_state, batch,
                         dim, seqlen, dstate, io_dtype, flags, workspace, workspace_bytes, stream, false);
}

int ssm_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                         const float* D, const void* z, const float* delta_bias, int softplus_flag,
                         void* out, float* last_state, int64_t batch, int64_t dim, int64_t seqlen,
                         int64_t dstate, int io_dtype, unsigned flags, void* stream) {
    return scan_fwd_impl("ssm_scan_fwd_noalloc", u, delta, A, B, C, D, z, delta_bias, softplus_flag, out, last_state,
                         batch, dim, seqlen, dstate, io_dtype, flags, nullptr, 0, stream, true);
}

size_t ssm_scan_fwd_noalloc_max_workspace(void) { return ssm::kNoAllocScratchBytes; }

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
    if (!mul_le(batch, dim, kMaxElems, &rows) || !mul_le(ssm::ceil_div(dim, 64), batch, kMaxBlocks, &blocks))
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
    const int64_t os = (flags & SSM_FLAG_OUT_F32) ? 4 : es;
    const int64_t sbytes = rows * dstate * 4;
    const int64_t abytes = dim * dstate * 4, bcbytes = batch * dstate * es;
    if (overlaps_any(out, rows * os, {state, x, delta, z, A, B, C, D},
                     {sbytes, rows * es, rows * es, rows * es, abytes, bcbytes, bcbytes, dim * 4}) ||
        overlaps_any(state, sbytes, {x, delta, z, A, B, C, D},
                     {rows * es, rows * es, rows * es, abytes, bcbytes, bcbytes, dim * 4}))
        return fail(SSM_ERR_BAD_SHAPE, "%s: out or state overlaps another tensor", fn);

    ssm::UpdateArgs a{state, x, delta, A, B, C, D, z, out, batch, dim, static_cast<int>(dstate),
                      (flags & SSM_FLAG_ZOH) != 0};
    a.out_f32 = (flags & SSM_FLAG_OUT_F32) != 0;
    const hipError_t e = ssm::launch_state_update(a, io_dtype == SSM_DTYPE_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

int ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* delta_bias, int softplus_flag, const void* dout, void* du, void* ddelta,
                 float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias, int64_t batch,
                 int64_t dim, int64_t seqlen, int64_t dstate, int io_dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
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
    // every output against every input and every other output
    const int64_t abytes = dim * dstate * 4, cbytes = dim * 4;
    const void* outs[] = {du, ddelta, z ? dz : nullptr, dA, dB, dC, dD, ddelta_bias};  // dz is unused without z
    const int64_t osz[] = {ib, ib, ib, abytes, bc * 4, bc * 4, cbytes, cbytes};
    for (int i = 0; i < 8; ++i) {
        const void* o = outs[i];
        if (!o) continue;
        if (overlaps_any(o, osz[i], {u, delta, dout, z, B, C, A, D, delta_bias},
                         {ib, ib, ib, ib, bc * es, bc * es, abytes, cbytes, cbytes}))
            return fail(SSM_ERR_BAD_SHAPE, "%s: a gradient overlaps an input", fn);
        for (int j = i + 1; j < 8; ++j)
            if (overlaps(o, osz[i], outs[j], osz[j]))
                return fail(SSM_ERR_BAD_SHAPE, "%s: gradient outputs overlap", fn);
    }

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
    const size_t scan_bytes = bwd_scan_part(ssm::scan_workspace_bytes(batch, dim, seqlen));
    if (int st = check_workspace(fn, workspace, workspace_bytes, scan_bytes + ssm::scan_bwd_extra_bytes(batch, dim, seqlen),
                                 {u, delta, z, B, C, dout, du, ddelta, dz, dA, dB, dC, dD, ddelta_bias, A, D, delta_bias},
                                 {ib, ib, ib, bc * es, bc * es, ib, ib, ib, ib, dim * dstate * 4, bc * 4, bc * 4, dim * 4,
                                  dim * 4, dim * dstate * 4, dim * 4, dim * 4}))
        return st;
    const hipError_t e = ssm::launch_scan_bwd(q, io_dtype == SSM_DTYPE_BF16, workspace,
                                              static_cast<char*>(workspace) + scan_bytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
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
    if (overlaps_any(out, elems * es, {x, weight, bias}, {elems * es, dim * width * 4, dim * 4}))
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
    if (overlaps_any(out, rows * es, {x, window, weight, bias}, {rows * es, wbytes, dim * width * 4, dim * 4}) ||
        overlaps_any(window, wbytes, {x, weight, bias}, {rows * es, dim * width * 4, dim * 4}))
        return fail(SSM_ERR_BAD_SHAPE, "%s: out, window or x overlap", fn);
    ssm::ConvArgs a{x, weight, bias, out, window, batch, dim, 1, static_cast<int>(width), silu_flag != 0};
    const hipError_t e = ssm::launch_conv_window_update(a, io_dtype == SSM_DTYPE_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

size_t ssm_ssd_scan_workspace_size(int64_t batch, int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate,
                                   int io_dtype) {
    int64_t bl, bh;
    if (batch < 1 || seqlen < 1 || seqlen > kSsdMaxSeqlen || heads < 1 || headdim < 16 || headdim > SSM_SSD_MAX_HEADDIM || headdim % 16 != 0 ||
        dstate < 16 || dstate > SSM_SSD_MAX_DSTATE || dstate % 16 != 0 ||
        (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16) || !mul_le(batch, seqlen, kMaxElems, &bl) ||
        !mul_le(batch, heads, kMaxBlocks, &bh))
        return 0;
    return ssm::ssd_workspace_bytes(ssm::ssd_plan(batch, seqlen, heads, io_dtype == SSM_DTYPE_BF16, true), batch,
                                    heads, headdim, dstate);
}

int ssm_ssd_scan(const void* x, const float* a, const void* b, const void* c, void* y, float* final_state,
                 int64_t batch, int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate, int64_t ngroups,
                 int io_dtype, unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ssm_ssd_scan";
    if (int s = check_dtype(io_dtype)) return s;
    if (flags & ~SSM_FLAG_OUT_F32)
        return fail(SSM_ERR_BAD_FLAGS, "%s: flag bits 0x%x do not apply (only SSM_FLAG_OUT_F32 does)", fn,
                    flags & ~SSM_FLAG_OUT_F32);
    CHECK_NONNULL(x);
    CHECK_NONNULL(a);
    CHECK_NONNULL(b);
    CHECK_NONNULL(c);
    CHECK_NONNULL(y);
    if (batch < 1 || seqlen < 1 || heads < 1 || ngroups < 1)
        return fail(SSM_ERR_BAD_SHAPE, "%s: batch=%lld seqlen=%lld heads=%lld ngroups=%lld must all be >= 1", fn,
                    (long long)batch, (long long)seqlen, (long long)heads, (long long)ngroups);
    if (heads % ngroups != 0)
        return fail(SSM_ERR_BAD_SHAPE, "%s: heads=%lld is not a multiple of ngroups=%lld", fn, (long long)heads,
                    (long long)ngroups);
    if (headdim < 16 || headdim > SSM_SSD_MAX_HEADDIM || headdim % 16 != 0)
        return fail(SSM_ERR_BAD_SHAPE, "%s: headdim=%lld must be a multiple of 16 in [16, %d]", fn, (long long)headdim,
                    SSM_SSD_MAX_HEADDIM);
    if (dstate < 16 || dstate > SSM_SSD_MAX_DSTATE || dstate % 16 != 0)
        return fail(SSM_ERR_BAD_SHAPE, "%s: dstate=%lld must be a multiple of 16 in [16, %d]", fn, (long long)dstate,
                    SSM_SSD_MAX_DSTATE);
    if (seqlen > kSsdMaxSeqlen)
        return fail(SSM_ERR_BAD_SHAPE, "%s: seqlen=%lld is above %lld", fn, (long long)seqlen, (long long)kSsdMaxSeqlen);
    if (heads > kSsdMaxRow / headdim || ngroups > kSsdMaxRow / dstate)
        return fail(SSM_ERR_BAD_SHAPE, "%s: heads x headdim (%lld x %lld) and ngroups x dstate (%lld x %lld) must be at "
                    "most %lld", fn, (long long)heads, (long long)headdim, (long long)ngroups, (long long)dstate,
                    (long long)kSsdMaxRow);
    int64_t bl, rows, elems, blg, bcel, bh, fsel;
    if (!mul_le(batch, seqlen, kMaxElems, &bl) || !mul_le(bl, heads, kMaxElems, &rows) ||
        !mul_le(rows, headdim, kMaxElems, &elems) || !mul_le(bl, ngroups, kMaxElems, &blg) ||
        !mul_le(blg, dstate, kMaxElems, &bcel) || !mul_le(batch, heads, kMaxBlocks, &bh) ||
        !mul_le(bh, headdim * dstate, kMaxElems, &fsel))
        return fail(SSM_ERR_BAD_SHAPE, "%s: sizes batch=%lld seqlen=%lld heads=%lld are too large", fn, (long long)batch,
                    (long long)seqlen, (long long)heads);
    CHECK_ALIGN(x);
    CHECK_ALIGN(a);
    CHECK_ALIGN(b);
    CHECK_ALIGN(c);
    CHECK_ALIGN(y);
    CHECK_ALIGN(final_state);
    const int64_t es = io_dtype == SSM_DTYPE_F32 ? 4 : 2;
    const int64_t ybytes = elems * ((flags & SSM_FLAG_OUT_F32) ? 4 : es);
    if (overlaps_any(y, ybytes, {x, a, b, c, final_state}, {elems * es, rows * 4, bcel * es, bcel * es, fsel * 4}))
        return fail(SSM_ERR_BAD_SHAPE, "%s: y overlaps another tensor argument", fn);
    if (final_state && overlaps_any(final_state, fsel * 4, {x, a, b, c}, {elems * es, rows * 4, bcel * es, bcel * es}))
        return fail(SSM_ERR_BAD_SHAPE, "%s: final_state overlaps another tensor argument", fn);
    // the plan: segments of the sequence, with their carries in the workspace; a NULL workspace runs unsplit
    const bool bf16 = io_dtype == SSM_DTYPE_BF16;
    ssm::SsdPlan plan = ssm::ssd_plan(batch, seqlen, heads, bf16, true);
    const size_t need = ssm::ssd_workspace_bytes(plan, batch, heads, headdim, dstate);
    if (!workspace) {
        if (workspace_bytes != 0)
            return fail(SSM_ERR_WORKSPACE, "%s: workspace is NULL but workspace_bytes is %zu", fn, workspace_bytes);
        plan = ssm::ssd_plan(batch, seqlen, heads, bf16, false);
    } else {
        CHECK_ALIGN(workspace);
        if (workspace_bytes < need)
            return fail(SSM_ERR_WORKSPACE, "%s: workspace_bytes=%zu < %zu (ssm_ssd_scan_workspace_size)", fn,
                        workspace_bytes, need);
        if (need && overlaps_any(workspace, need, {x, a, b, c, y, final_state},
                                 {elems * es, rows * 4, bcel * es, bcel * es, ybytes, fsel * 4}))
            return fail(SSM_ERR_WORKSPACE, "%s: the workspace overlaps a tensor argument", fn);
    }
    ssm::SsdArgs q{x, a, b, c, y, final_state, batch, seqlen, heads, headdim, dstate, ngroups,
                   (flags & SSM_FLAG_OUT_F32) != 0, plan, nullptr, nullptr};
    const hipError_t e = ssm::launch_ssd_scan(q, bf16, plan.segments > 1 ? workspace : nullptr,
                                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

size_t ssm_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t seqlen) {
    if (ssm_scan_fwd_workspace_size(batch, dim, seqlen) == 0) return 0;
    return bwd_scan_part(ssm::scan_workspace_bytes(batch, dim, seqlen)) + ssm::scan_bwd_extra_bytes(batch, dim, seqlen);
}

int ssm_workspace_check(const void* workspace, void* stream) {
    const char* fn = "ssm_workspace_check";
    CHECK_NONNULL(workspace);
    CHECK_ALIGN(workspace);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e = hipStreamSynchronize(hs);
    uint32_t v = 0;
    if (e == hipSuccess) e = hipMemcpy(&v, workspace, sizeof(v), hipMemcpyDeviceToHost);
    if (e == hipSuccess && v) {
        const uint32_t zero = 0;
        e = hipMemcpy(const_cast<void*>(workspace), &zero, sizeof(zero), hipMemcpyHostToDevice);
    }
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    if (v)
        return fail(SSM_ERR_DEVICE_WAIT, "%s: a scan on this workspace timed out waiting for another workgroup "
                                         "(flags 0x%x); its outputs are not valid, and the workspace must be "
                                         "zero-filled again before it is reused", fn, v);
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
        case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE";
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
