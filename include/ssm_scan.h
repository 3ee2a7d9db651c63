/*
 * ssm_scan.h - C ABI of the MI355X (gfx950) selective-scan library, libssmscan.so.
 *
 * The library implements the hot path of the Mamba S6 layer: the fused selective scan over a
 * whole sequence and the one-token state update used for decoding. The operations are defined
 * on these pages:
 *   - "Beyond attention with Mamba, state space models and hybrids", section 3 "Selectivity"
 *     (the selective recurrence h_t = exp(D_t a) h_{t-1} + D_t b_t x_t, y_t = c_t^T h_t),
 *     section 4 "The Mamba block" (the step D = softplus(dt_proj(.)) with the projection's bias
 *     inside the softplus; decay exp(step*a) and write step*b*u; the readout; the skip u*D; the
 *     gate y*SiLU(z); the result cast back to u's dtype), section 6 "The scan" (the fused kernel
 *     keeps the per-step states on chip and writes back only y) and section 7 "Generation with a
 *     state of fixed size" (mixer_step: the one-token update of h);
 *   - "Module 19: State-Space Models (Mamba)", sections "The Math: The State-Space Recurrence"
 *     (zero-order hold Abar = exp(Delta A); the Euler input gain Bbar ~ Delta B that the fused
 *     kernel uses) and "The Parallel Scan" (the associative composition of affine steps).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (memory on the current HIP device), allocated,
 *     owned and freed by the caller. The library keeps no pointer after a call returns.
 *   - Layouts are dense, row-major, last index fastest. Every pointer must be 16-byte aligned.
 *   - io_dtype (ssm_dtype_t) selects the element type of u/x, delta, z, B, C and out together:
 *     SSM_DTYPE_F32 (float) or SSM_DTYPE_BF16 (bfloat16 bit patterns, 2 bytes). A, D,
 *     delta_bias, last_state and state are always fp32. Arithmetic is fp32; bf16 outputs are
 *     rounded to nearest even.
 *   - dstate (N) must be in [1, 16]; batch, dim and seqlen must be >= 1.
 *   - stream is a hipStream_t (NULL = the default stream). Work is enqueued on it and the call
 *     returns without synchronising; results are visible after the stream is synchronised.
 *   - Every argument is validated before any HIP call; an invalid call returns a nonzero
 *     ssm_status_t, launches nothing and sets the thread's last-error message. Launch failures
 *     return SSM_ERR_HIP. A fault inside a kernel surfaces at the caller's next synchronisation.
 *   - No exception or abort crosses the ABI. Calls on different streams may run concurrently.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 4
#define SSM_MAX_DSTATE 16
#define SSM_MAX_CONV_WIDTH 8
#define SSM_SSD_MAX_DSTATE 128  /* ssm_ssd_scan: dstate is a multiple of 16 up to this */
#define SSM_SSD_MAX_HEADDIM 64  /* ssm_ssd_scan: headdim is a multiple of 16 up to this */

typedef enum ssm_dtype { SSM_DTYPE_F32 = 0, SSM_DTYPE_BF16 = 1 } ssm_dtype_t;

typedef enum ssm_status {
    SSM_OK = 0,
    SSM_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
    SSM_ERR_BAD_SHAPE = 2,    /* a size is out of range (or their product overflows) */
    SSM_ERR_BAD_DTYPE = 3,    /* io_dtype is not an ssm_dtype_t value */
    SSM_ERR_MISALIGNED = 4,   /* a pointer is not 16-byte aligned */
    SSM_ERR_HIP = 5,          /* the HIP runtime reported an error (message has the detail) */
    SSM_ERR_DEVICE_WAIT = 6,  /* a scan kernel's bounded cross-workgroup wait timed out (reported by
                                 ssm_workspace_check); that call's outputs are not valid */
    SSM_ERR_BAD_FLAGS = 7,    /* a flags argument has bits that are not SSM_FLAG_* values */
    SSM_ERR_WORKSPACE = 8     /* the workspace is NULL, smaller than the size query says, or overlaps
                                 a tensor argument */
} ssm_status_t;

/*
 * Flags of the _ex entry points.
 * SSM_FLAG_ZOH: discretise the input with the exact zero-order hold instead of the Euler gain:
 *   Bbar u = (exp(Delta A) - 1) / A * B * u   (-> Delta B u as Delta A -> 0)
 * ("Module 19: State-Space Models (Mamba)", The Math: The State-Space Recurrence, the discretised
 * input matrix; "Beyond attention with Mamba, state space models and hybrids", section 3, where the
 * exact form is compared with the Euler gain). The decay exp(Delta A) is the same in both modes.
 */
#define SSM_FLAG_ZOH 1u
/*
 * SSM_FLAG_OUT_F32: write `out` as fp32 whatever io_dtype is (the inputs keep io_dtype). The result is
 * the one the bf16 output is rounded from: with io_dtype = SSM_DTYPE_BF16, the default output is this
 * value rounded to nearest even. (The pages cast the result back to the input's dtype, "Beyond
 * attention with Mamba, state space models and hybrids", section 4; this flag leaves the cast to the
 * caller.)
 */
#define SSM_FLAG_OUT_F32 2u

/*
 * Selective scan forward over a whole sequence, from a zero initial state.
 *
 * For every batch row b, channel d and token t (t ascending), with s = delta_bias[d] (0 if NULL):
 *   Delta   = softplus(delta[b,d,t] + s)  if softplus_flag != 0,  else  delta[b,d,t] + s
 *   h[n]    = exp(Delta * A[d,n]) * h[n] + Delta * B[b,t,n] * u[b,d,t]      (n < dstate; h starts at 0)
 *   y       = sum_n C[b,t,n] * h[n]  +  D[d] * u[b,d,t]                    (skip omitted if D is NULL)
 *   out     = y * z * sigmoid(z) with z = z[b,d,t]                          (gate omitted if z is NULL)
 * and after the last token last_state[b,d,n] = h[n] (not written if last_state is NULL).
 *
 * Arguments (shapes in elements):
 *   u, delta, z, out : [batch, dim, seqlen], io_dtype. out may not alias any input.
 *   A                : [dim, dstate] fp32 (negative entries give a decaying state).
 *   B, C             : [batch, seqlen, dstate], io_dtype; shared by every channel of a batch row.
 *   D, delta_bias    : [dim] fp32, nullable.
 *   last_state       : [batch, dim, dstate] fp32, nullable.
 * The per-step states are never written to memory; only out and last_state are.
 *
 * Workspace (the caller's): workgroups handle 64-token segments of 64 channels and hand segment
 * states to their successors through it. Its size comes from ssm_scan_fwd_workspace_size(); it must
 * be zero-filled once before its first use (after that the kernels leave it ready for the next call
 * on any shape, so it is never cleared again), and it must not be used by two calls that may run at
 * the same time (calls on one stream run one after another). The library itself allocates nothing
 * and never synchronises. If a call's bounded cross-workgroup wait times out, the call still returns
 * SSM_OK and its outputs are invalid: ssm_workspace_check() reports it, and the workspace must then
 * be zero-filled again. The kernels keep a launch tag in the workspace, so a call captured in a HIP
 * graph stays valid on every replay.
 */
int ssm_scan_fwd(const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *delta_bias, int softplus_flag,
                 void *out, float *last_state,
                 int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int io_dtype,
                 void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace that ssm_scan_fwd needs for these sizes (about 8.5 KB per 64 channels per 64
 * tokens per batch row), or 0 if the sizes are invalid. Makes no HIP call. */
size_t ssm_scan_fwd_workspace_size(int64_t batch, int64_t dim, int64_t seqlen);

/* ssm_scan_fwd with flags (SSM_FLAG_ZOH, SSM_FLAG_OUT_F32, or 0); ssm_scan_fwd(...) is ssm_scan_fwd_ex(..., 0, workspace,
 * workspace_bytes, stream). Unknown flag bits return SSM_ERR_BAD_FLAGS. */
int ssm_scan_fwd_ex(const void *u, const void *delta, const float *A, const void *B, const void *C,
                    const float *D, const void *z, const float *delta_bias, int softplus_flag,
                    void *out, float *last_state,
                    int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int io_dtype,
                    unsigned flags, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssm_scan_fwd_ex for callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, on a workspace the library holds instead of
 * a caller's. That workspace is a device array of ssm_scan_fwd_noalloc_max_workspace() bytes (64 MiB),
 * one per GPU the library runs on, held until the process ends; the first call on a device clears it
 * with a kernel on `stream`. The call allocates nothing and does not synchronise. A problem whose
 * workspace (ssm_scan_fwd_workspace_size) exceeds the array returns SSM_ERR_WORKSPACE and launches
 * nothing. All calls on one GPU share the array: calls that may overlap in time on one GPU (different
 * streams) race and give wrong results; calls on one stream are ordered. A cross-workgroup wait that
 * times out is recorded in the array but not reported (no call reads it back); a caller that needs
 * that report uses ssm_scan_fwd with ssm_workspace_check.
 */
int ssm_scan_fwd_noalloc(const void *u, const void *delta, const float *A, const void *B, const void *C,
                         const float *D, const void *z, const float *delta_bias, int softplus_flag,
                         void *out, float *last_state,
                         int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int io_dtype,
                         unsigned flags, void *stream);

/* Bytes of the device array ssm_scan_fwd_noalloc uses as its workspace. Makes no HIP call. */
size_t ssm_scan_fwd_noalloc_max_workspace(void);

/*
 * Backward of ssm_scan_fwd (Euler input gain): given dout = dL/dout, the gradients of L with respect
 * to every input. The states are recomputed, not stored ("Beyond attention with Mamba, state space
 * models and hybrids", section 6): a forward pass writes the state entering every 16-token block to
 * the workspace, and the adjoint lambda_t = C_t dy_t + exp(Delta_{t+1} A) lambda_{t+1}
 * (dy_t = dout_t SiLU(z_t)) runs backwards through each block from there.
 * Inputs: as ssm_scan_fwd (u, delta, A, B, C, D, z, delta_bias, softplus_flag, sizes, io_dtype), and
 *   dout                       [batch, dim, seqlen] io_dtype.
 * Outputs (all written, never accumulated into):
 *   du, ddelta                 [batch, dim, seqlen] io_dtype (ddelta is the gradient of the raw delta,
 *                              through the softplus when softplus_flag is set);
 *   dz                         [batch, dim, seqlen] io_dtype; required when z is given, unused otherwise;
 *   dA                         [dim, dstate] fp32;  dB, dC [batch, seqlen, dstate] fp32 (summed over dim);
 *   dD, ddelta_bias            [dim] fp32, nullable (written when given: the gradient at the given D or
 *                              bias, or at 0 when that input is NULL).
 * Sums over channels and tokens are computed in a fixed order (no atomics): results are reproducible.
 * Workspace: ssm_scan_bwd_workspace_size() bytes, under the same contract as ssm_scan_fwd's (zero-filled
 * once before first use, one call at a time); about 12 bytes per (batch, channel, token) plus 8 bytes
 * per (channel group of 64, batch, token, state) beyond the forward's.
 */
int ssm_scan_bwd(const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *delta_bias, int softplus_flag, const void *dout,
                 void *du, void *ddelta, float *dA, float *dB, float *dC, float *dD, void *dz,
                 float *ddelta_bias, int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int io_dtype,
                 void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace that ssm_scan_bwd needs for these sizes, or 0 if the sizes are invalid. */
size_t ssm_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t seqlen);

/*
 * One decode step: the scan's recurrence for a single token, with the state carried by the
 * caller and updated in place. For every b, d:
 *   Delta   = softplus(delta[b,d])                      (always; fold any bias into delta)
 *   state[b,d,n] = exp(Delta * A[d,n]) * state[b,d,n] + Delta * B[b,n] * x[b,d]
 *   y       = sum_n C[b,n] * state[b,d,n] + D[d] * x[b,d]          (skip omitted if D is NULL)
 *   out[b,d] = y * z * sigmoid(z), z = z[b,d]                       (gate omitted if z is NULL)
 *
 * Arguments: state [batch, dim, dstate] fp32 (read and written); x, delta, z, out [batch, dim]
 * io_dtype; A [dim, dstate] fp32; B, C [batch, dstate] io_dtype; D [dim] fp32 (nullable);
 * z nullable. out may not alias state or an input.
 * Iterating it over the tokens of a sequence from a zero state reproduces ssm_scan_fwd with
 * softplus_flag = 1 and delta_bias = NULL.
 */
int ssm_state_update(float *state, const void *x, const void *delta, const float *A, const void *B,
                     const void *C, const float *D, const void *z, void *out,
                     int64_t batch, int64_t dim, int64_t dstate, int io_dtype, void *stream);

/* ssm_state_update with flags (SSM_FLAG_ZOH, SSM_FLAG_OUT_F32, or 0); with SSM_FLAG_ZOH the steps reproduce
 * ssm_scan_fwd_ex(..., SSM_FLAG_ZOH, ...). Unknown flag bits return SSM_ERR_BAD_FLAGS. */
int ssm_state_update_ex(float *state, const void *x, const void *delta, const float *A, const void *B,
                        const void *C, const float *D, const void *z, void *out,
                        int64_t batch, int64_t dim, int64_t dstate, int io_dtype, unsigned flags, void *stream);

/*
 * Causal depthwise convolution, then SiLU: the step that produces the scan's input u in the Mamba
 * block ("Module 19: State-Space Models (Mamba)", The Causal Convolution and The Math: Six Stages;
 * "Beyond attention with Mamba, state space models and hybrids", section 4, the Mixer's conv1d
 * with padding width-1 cropped to the sequence). For every batch row b, channel d and token t:
 *   pre = bias[d] + sum_{k < width} weight[d, k] * x[b, d, t - (width-1) + k]   (x before t = 0 is 0)
 *   out[b, d, t] = silu_flag ? pre * sigmoid(pre) : pre
 * Each channel has its own taps; output t reads no input after t.
 * Arguments: x, out [batch, dim, seqlen] io_dtype (out may not alias x); weight [dim, width] fp32;
 * bias [dim] fp32, nullable; width in [1, SSM_MAX_CONV_WIDTH] (Mamba uses 4).
 */
int ssm_causal_conv1d(const void *x, const float *weight, const float *bias, int silu_flag, void *out,
                      int64_t batch, int64_t dim, int64_t seqlen, int64_t width, int io_dtype, void *stream);

/*
 * One decode step of the convolution ("Beyond attention with Mamba, state space models and
 * hybrids", section 7, mixer_step): the window of the last `width` inputs of each (b, d) shifts by
 * one, x enters at the end, and
 *   out[b, d] = act(bias[d] + sum_k weight[d, k] * window[b, d, k])   (act = SiLU if silu_flag)
 * window [batch, dim, width] fp32 is read and written in place (zeros before the first token);
 * x, out [batch, dim] io_dtype. Steps from a zero window reproduce ssm_causal_conv1d token by token.
 */
int ssm_conv_window_update(float *window, const void *x, const float *weight, const float *bias, int silu_flag,
                           void *out, int64_t batch, int64_t dim, int64_t width, int io_dtype, void *stream);

/*
 * Synchronise `stream`, then report whether a scan or backward call on `workspace` since the last check
 * hit the limit of a cross-workgroup wait (SSM_ERR_DEVICE_WAIT; that call's outputs are invalid and
 * the workspace must be zero-filled again before reuse). Clears the recorded flag. Every wait inside
 * the kernels is bounded, so a launch always completes; this call tells whether one completed without
 * its carry. Returns SSM_OK otherwise.
 */
int ssm_workspace_check(const void *workspace, void *stream);

/*
 * Mamba-2's scan with a scalar decay per head ("Beyond attention with Mamba, state space models and
 * hybrids", section 8, Mamba-2: the same model as attention). For every batch row b and head h, with a
 * state H of headdim x dstate numbers that starts at zero, token by token:
 *   H = exp(a[b,t,h]) H + x[b,t,h,:] b[b,t,g,:]^T        (g = h / (heads / ngroups))
 *   y[b,t,h,p] = sum_n H[p,n] c[b,t,g,n]
 * computed by the page's chunked form (attention masked by the decay inside chunks of tokens, the
 * recurrence between chunks) on the matrix cores; with bf16 inputs the intermediate fp32 values that
 * feed a second product are split into two bf16 parts, so the accuracy stays close to fp32.
 * Arguments (device pointers; the caller allocates and owns every buffer):
 *   x            [batch, seqlen, heads, headdim] io_dtype: the stream, already multiplied by its step;
 *   a            [batch, seqlen, heads] fp32: the step times the head's A (any real; <= 0 decays);
 *   b, c         [batch, seqlen, ngroups, dstate] io_dtype: each group serves heads / ngroups heads;
 *   y            [batch, seqlen, heads, headdim] io_dtype, or fp32 with SSM_FLAG_OUT_F32 (may not alias
 *                an input);
 *   final_state  [batch, heads, headdim, dstate] fp32, the state after the last token; nullable.
 *   workspace    scratch of ssm_ssd_scan_workspace_size() bytes (16-byte aligned; not kept between
 *                calls, needs no initialisation; may not overlap any tensor argument), or NULL with
 *                workspace_bytes 0.
 * headdim and dstate are multiples of 16 up to SSM_SSD_MAX_HEADDIM and SSM_SSD_MAX_DSTATE; heads is a
 * multiple of ngroups; seqlen is at most 2^35; heads x headdim and ngroups x dstate are at most 2^24. flags: 0 or SSM_FLAG_OUT_F32 (other bits return SSM_ERR_BAD_FLAGS). Every
 * argument is checked before any HIP call; a workspace smaller than the size query says returns
 * SSM_ERR_WORKSPACE. The call allocates nothing and does not synchronise.
 * Where batch x heads is small, each (batch row, head)'s sequence is cut into up to 16 segments of whole
 * chunks: one kernel computes each segment's own contribution to the state into the workspace, a second
 * turns them in order into the state entering each segment, a third computes the outputs, every segment
 * in parallel. With a NULL workspace (or where the size query returns 0) one workgroup per (batch row,
 * head) walks the whole sequence in order. The two forms differ only in rounding. Calls that may run at
 * the same time need workspaces of their own.
 */
int ssm_ssd_scan(const void *x, const float *a, const void *b, const void *c, void *y, float *final_state,
                 int64_t batch, int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate, int64_t ngroups,
                 int io_dtype, unsigned flags, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace ssm_ssd_scan takes for this shape (0: the shape runs unsplit and needs none; also
 * 0 for sizes ssm_ssd_scan rejects). Makes no HIP call.
 */
size_t ssm_ssd_scan_workspace_size(int64_t batch, int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate,
                                   int io_dtype);

/*
 * Tokens per segment (one workgroup's share of the sequence, for 64 channels of one batch row) that
 * ssm_scan_fwd uses for this shape: 64 (4 waves of 16 tokens). It sets the workspace size and the
 * number of cross-workgroup carries. Returns 0 for sizes < 1. Makes no HIP call.
 */
int ssm_scan_segment_tokens(int64_t batch, int64_t dim, int64_t seqlen);

/*
 * Number of polls a scan's cross-workgroup wait may take before it gives up and records
 * SSM_ERR_DEVICE_WAIT (each poll sleeps briefly; the default, about 0.1 s in all, applies when
 * polls <= 0). Applies to launches made after the call, in this process. Returns the previous
 * value. A small limit makes the timeout path observable: the kernels still finish, and
 * ssm_workspace_check reports the timed-out launch.
 */
int ssm_set_wait_limit(int polls);

/* Human-readable name of a status code (static storage). */
const char *ssm_status_string(int status);

/* Detail of the last failed call on the calling thread ("" if none); valid until the thread's
 * next call into the library. */
const char *ssm_last_error_message(void);

/* SSM_ABI_VERSION of the loaded library. */
int ssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
