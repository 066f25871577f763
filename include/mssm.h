/*
 * mssm.h -- C ABI of libmssm.so, the MI355X (gfx950) selective state-space
 * scan library.
 *
 * Seven operations, each defined by the pages it cites:
 *
 *   mssm_selective_scan_fwd  the S6 selective scan over a whole sequence
 *                            (mssm_selective_scan_fwd_save: the same, also
 *                            keeping the states the backward starts from);
 *   mssm_selective_scan_zoh_fwd  the same scan with the zero-order-hold
 *                            input term;
 *   mssm_selective_scan_fused_fwd  the same scan with its input front end
 *                            (causal conv1d + SiLU, softplus step) fused in;
 *   mssm_selective_scan_bwd  the gradients of that scan (training;
 *                            mssm_selective_scan_bwd_saved: from the states
 *                            mssm_selective_scan_fwd_save kept);
 *   mssm_state_update        one decode token of the same recurrence;
 *   mssm_ssd_chunk_fwd       the Mamba-2 SSD (scalar transition per head),
 *                            computed chunk by chunk;
 *   mssm_ssd_state_update    one Mamba-2 decode token of that recurrence.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked (device) are device pointers in the current HIP device's
 *   memory; every tensor is dense and contiguous in the layout given (row-
 *   major, last index fastest).  The library does not allocate, free, or
 *   synchronise: all work is enqueued on `stream` (a hipStream_t; NULL means
 *   the default stream) and the call returns as soon as it is enqueued.
 * - The caller owns every buffer.  Inputs are only read; outputs are only
 *   written; `state` of mssm_state_update is read and then overwritten.
 *   Outputs must not alias inputs (except `state`, which is in place).
 * - `dtype` selects the storage type of the per-token tensors (u, delta, z,
 *   B, C, x, dt, y): MSSM_F32 (IEEE binary32) or MSSM_BF16 (bfloat16).  A, D,
 *   h0, h_final and `state` are always float32; all arithmetic and the
 *   recurrent state are float32; a bf16 output is rounded to nearest-even.
 * - Errors: argument problems are reported synchronously, before anything is
 *   enqueued, as a negative MSSM_ERR_* code; mssm_last_error() then returns a
 *   message for the calling thread.  A launch failure returns
 *   MSSM_ERR_LAUNCH.  Faults during execution surface at the caller's next
 *   synchronisation of `stream`.  MSSM_OK (0) means the work was enqueued.
 * - Every base pointer must be aligned to 16 bytes (MSSM_ERR_ALIGN).
 * - Zero-length sequences are valid: nothing is launched for the scan
 *   itself; h_final (if requested) receives h0, or zeros.
 * - The functions are stateless and may be called from several threads.
 */
#ifndef MSSM_H
#define MSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MSSM_F32 = 0, MSSM_BF16 = 1 } mssm_dtype;

/* Longest sequence the S6 entry points (forward, fused, zero-order hold,
 * backward) accept: 2^31 - 2^16 tokens, so that token indices rounded up to
 * whole chunks stay within 32-bit signed integers. */
#define MSSM_MAX_SEQLEN 2147418112LL

enum {
    MSSM_OK = 0,
    MSSM_ERR_NULL = -1,         /* a required pointer is NULL                 */
    MSSM_ERR_SHAPE = -2,        /* a dimension is negative or inconsistent    */
    MSSM_ERR_DTYPE = -3,        /* dtype is not an mssm_dtype value           */
    MSSM_ERR_UNSUPPORTED = -4,  /* a size outside what the kernels implement  */
    MSSM_ERR_ALIGN = -5,        /* a base pointer is not 16-byte aligned      */
    MSSM_ERR_WORKSPACE = -6,    /* workspace missing or too small             */
    MSSM_ERR_LAUNCH = -7        /* the HIP launch itself failed               */
};

/*
 * S6 selective scan (forward).
 *
 * Defined by: "Mamba Architecture Details" page, "Selective State Space
 * Mechanism / How S6 Works" -- input-dependent delta, B, C and the update
 * h(t) = discretize(A, delta(t)) h(t-1) + delta(t) B(t) x(t), y(t) = C(t) h(t);
 * the "State-Space Model Optimization Patterns" page, section 7 -- the transition is
 * exp(delta A), elementwise because A is diagonal; section 6 -- the skip
 * term D x; section 3 -- the output gate, here silu(z) = z / (1 + exp(-z)).
 * For every batch row b, channel d and state index n (h starts at h0, or 0):
 *
 *   h[n] <- exp(delta[b,d,t] * A[d,n]) * h[n] + delta[b,d,t] * u[b,d,t] * B[b,n,t]
 *   y[b,d,t] = (sum_n C[b,n,t] * h[n] + D[d] * u[b,d,t]) * silu(z[b,d,t])
 *
 * The input term is the first-order (Euler) form delta*B*u; delta is used as
 * given (it must already be positive: no softplus or bias is applied).
 *
 *   u, delta   (device) [batch, d_inner, seqlen]  dtype
 *   A          (device) [d_inner, d_state]        float32 (any real; Mamba uses A < 0)
 *   Bm, Cm     (device) [batch, d_state, seqlen]  dtype, shared by all channels
 *   Dskip      (device) [d_inner] float32, NULL => no skip term
 *   z          (device) [batch, d_inner, seqlen]  dtype, NULL => no gate
 *   h0         (device) [batch, d_inner, d_state] float32, NULL => zero start
 *   y          (device) [batch, d_inner, seqlen]  dtype, output
 *   h_final    (device) [batch, d_inner, d_state] float32, NULL => not written
 *
 * Limits: 1 <= d_state <= 64 and seqlen <= MSSM_MAX_SEQLEN
 * (MSSM_ERR_UNSUPPORTED otherwise); batch, d_inner, seqlen >= 0;
 * batch*d_inner*seqlen < 2^62.
 */
int mssm_selective_scan_fwd(const void* u, const void* delta, const float* A,
                            const void* Bm, const void* Cm, const float* Dskip,
                            const void* z, const float* h0, void* y, float* h_final,
                            int64_t batch, int64_t d_inner, int64_t seqlen,
                            int64_t d_state, mssm_dtype dtype, void* stream);

/*
 * S6 selective scan with the zero-order-hold input term (forward).
 *
 * Defined by: the "State-Space Model Optimization Patterns" page, section 7,
 * which discretises B as (A_bar - I) A^-1 B with A_bar = exp(delta A); with a
 * diagonal A that is, per state, (exp(delta A[d,n]) - 1) / A[d,n] * B, the
 * exact discretisation of dh/dt = A h + B u for an input held over the step.
 * Everything else is mssm_selective_scan_fwd:
 *
 *   h[n] <- exp(delta*A[d,n]) * h[n] + (exp(delta*A[d,n]) - 1) / A[d,n] * u * B[b,n,t]
 *
 * with the term's limit delta * u * B at A[d,n] = 0 (computed without
 * cancellation for small delta*A).  Arguments, layouts, limits and errors are
 * those of mssm_selective_scan_fwd.
 */
int mssm_selective_scan_zoh_fwd(const void* u, const void* delta, const float* A,
                                const void* Bm, const void* Cm, const float* Dskip,
                                const void* z, const float* h0, void* y, float* h_final,
                                int64_t batch, int64_t d_inner, int64_t seqlen,
                                int64_t d_state, mssm_dtype dtype, void* stream);

/*
 * S6 selective scan with its front end fused in (forward).
 *
 * Defined by: "Mamba Architecture Details" page, "Hardware-Aware
 * Implementation / CUDA Kernel Optimizations" -- discretisation, the
 * recurrence and the 1-D convolution fused in one kernel; "Model
 * Configuration" -- d_conv (4 in the configurations); "Mamba Block
 * Structure" -- the causal convolution and SiLU that produce the SSM input;
 * "Initialization Strategy" -- the step is a softplus of a projection plus
 * a bias.  For every (b, d, t), with xx = concat(conv_init[b,d,:], x[b,d,:])
 * (conv_init taken as zeros when NULL):
 *
 *   u[b,d,t]     = silu(sum_{k<d_conv} conv_w[d,k] * xx[b,d,t+k] + conv_b[d])
 *   delta[b,d,t] = softplus(delta_raw[b,d,t] + delta_bias[d]),  softplus(v) = log(1 + e^v)
 *
 * then exactly mssm_selective_scan_fwd on (u, delta, A, Bm, Cm, Dskip, z, h0),
 * the skip term using this u.  The last d_conv - 1 entries of x are the
 * conv_init of a following call (together with h_final as its h0).
 *
 *   x, delta_raw (device) [batch, d_inner, seqlen] dtype
 *   conv_w     (device) [d_inner, d_conv] float32
 *   conv_b     (device) [d_inner] float32, NULL => 0
 *   conv_init  (device) [batch, d_inner, d_conv - 1] dtype, NULL => zeros
 *   delta_bias (device) [d_inner] float32, NULL => 0
 *   the rest   as mssm_selective_scan_fwd
 *
 * Limits: 1 <= d_conv <= 4, 1 <= d_state <= 64 and seqlen <= MSSM_MAX_SEQLEN
 * (MSSM_ERR_UNSUPPORTED).
 */
int mssm_selective_scan_fused_fwd(const void* x, const float* conv_w, const float* conv_b,
                                  const void* conv_init, const void* delta_raw,
                                  const float* delta_bias, const float* A, const void* Bm,
                                  const void* Cm, const float* Dskip, const void* z,
                                  const float* h0, void* y, float* h_final, int64_t batch,
                                  int64_t d_inner, int64_t seqlen, int64_t d_state,
                                  int64_t d_conv, mssm_dtype dtype, void* stream);

/*
 * Backward of the S6 scan: the gradients of the loss
 *     sum(dout * y) + sum(dh_final * h_final)
 * with respect to every input of mssm_selective_scan_fwd.
 *
 * Defined by: the recurrence of mssm_selective_scan_fwd (same pages), and
 * "State-Space Model Optimization Patterns" page, section 4 -- the training
 * pass recomputes the forward states rather than storing them.  With
 * g = dout * silu(z) (dout without a gate), a_t = exp(delta_t A) and the
 * adjoint lambda_t = dL/dh_t:
 *   lambda_t = a_{t+1} lambda_{t+1} + g_t C_t   (dh_final at the last token, or 0)
 *   du_t = g_t D + sum_n lambda_t delta_t B_t;  ddelta_t = sum_n lambda_t (A a_t h_{t-1} + u_t B_t)
 *   dA = sum_{b,t} lambda_t delta_t a_t h_{t-1};  dB_t = sum_d lambda_t delta_t u_t;
 *   dC_t = sum_d g_t h_t;  dD = sum_{b,t} g_t u_t;  dz_t = dout_t y_t silu'(z_t);  dh0 = a_0 lambda_0.
 *
 *   u, delta, A, Bm, Cm, Dskip, z, h0: as mssm_selective_scan_fwd
 *   dout       (device) [batch, d_inner, seqlen] dtype, gradient of y
 *   dh_final   (device) [batch, d_inner, d_state] float32, NULL => 0
 *   du, ddelta (device) [batch, d_inner, seqlen] dtype, outputs
 *   dA         (device) [d_inner, d_state] float32, output (summed over batch)
 *   dB, dC     (device) [batch, d_state, seqlen] float32, outputs (summed over channels)
 *   dD         (device) [d_inner] float32, NULL => not computed
 *   dz         (device) [batch, d_inner, seqlen] dtype; required when z is given
 *   dh0        (device) [batch, d_inner, d_state] float32, NULL => not written
 *   workspace  (device) at least mssm_selective_scan_bwd_workspace_size(...)
 *              bytes (the state at every chunk start, and per-block partial
 *              sums of dB and dC); caller-owned, contents unspecified
 *
 * dA and dD are accumulated with atomics, so their last bits can vary from
 * call to call; the other outputs are deterministic.  With seqlen = 0, dh0
 * receives dh_final (or zeros) and dA, dD zeros.  Limits: 1 <= d_state <= 64
 * and seqlen <= MSSM_MAX_SEQLEN.
 */
size_t mssm_selective_scan_bwd_workspace_size(int64_t batch, int64_t d_inner, int64_t seqlen,
                                              int64_t d_state);
int mssm_selective_scan_bwd(const void* u, const void* delta, const float* A, const void* Bm,
                            const void* Cm, const float* Dskip, const void* z, const float* h0,
                            const void* dout, const float* dh_final, void* du, void* ddelta,
                            float* dA, float* dB, float* dC, float* dD, void* dz, float* dh0,
                            int64_t batch, int64_t d_inner, int64_t seqlen, int64_t d_state,
                            void* workspace, size_t workspace_bytes, mssm_dtype dtype,
                            void* stream);

/*
 * The training pair: a forward scan that keeps the states the backward starts
 * its chunks from, and the backward that uses them instead of re-running the
 * recurrence over the whole sequence first.
 *
 * Defined by: the same recurrence and gradients as mssm_selective_scan_fwd and
 * mssm_selective_scan_bwd; "State-Space Model Optimization Patterns" page,
 * section 4 -- the forward saves states at chunk boundaries and the backward
 * recomputes within each chunk from them.
 *
 * mssm_selective_scan_fwd_save takes the arguments of mssm_selective_scan_fwd
 * plus `workspace` / `workspace_bytes`: a (device) buffer of at least
 * mssm_selective_scan_bwd_workspace_size(batch, d_inner, seqlen, d_state)
 * bytes, 16-byte aligned, owned by the caller.  It writes y and h_final
 * exactly as mssm_selective_scan_fwd does (bit for bit), and the state at
 * every backward chunk start into the front of the workspace.
 *
 * mssm_selective_scan_bwd_saved takes the arguments of mssm_selective_scan_bwd
 * and returns the same gradients (bit for bit, dA and dD up to the order of
 * their atomic sums), provided its `workspace` still holds what
 * mssm_selective_scan_fwd_save wrote there for the same u, delta, A, Bm, h0
 * and sizes.  Anything else in the workspace gives wrong gradients; this is
 * not checked.  Errors and limits: as the two calls they mirror; in addition
 * the saved states of one batch row (4 * d_state * d_inner * seqlen / 16
 * bytes, / 8 when d_state > 16) must stay below 2 GiB
 * (MSSM_ERR_UNSUPPORTED).
 */
int mssm_selective_scan_fwd_save(const void* u, const void* delta, const float* A,
                                 const void* Bm, const void* Cm, const float* Dskip,
                                 const void* z, const float* h0, void* y, float* h_final,
                                 int64_t batch, int64_t d_inner, int64_t seqlen,
                                 int64_t d_state, void* workspace, size_t workspace_bytes,
                                 mssm_dtype dtype, void* stream);
int mssm_selective_scan_bwd_saved(const void* u, const void* delta, const float* A,
                                  const void* Bm, const void* Cm, const float* Dskip,
                                  const void* z, const float* h0, const void* dout,
                                  const float* dh_final, void* du, void* ddelta, float* dA,
                                  float* dB, float* dC, float* dD, void* dz, float* dh0,
                                  int64_t batch, int64_t d_inner, int64_t seqlen,
                                  int64_t d_state, void* workspace, size_t workspace_bytes,
                                  mssm_dtype dtype, void* stream);

/*
 * Decode: one token of the same recurrence, state updated in place.
 *
 * Defined by: "Mamba Architecture Details" page, "Hardware-Aware
 * Implementation / Parallel Algorithm", sequential (inference) mode -- a
 * constant-size state updated per token, h = A h + B x_t, then y_t = C h
 * read from the UPDATED state; the transition, skip and gate as above.
 *
 *   state      (device) [batch, d_inner, d_state] float32, read and overwritten
 *   u, delta   (device) [batch, d_inner] dtype
 *   A          (device) [d_inner, d_state] float32
 *   Bm, Cm     (device) [batch, d_state] dtype
 *   Dskip      (device) [d_inner] float32, NULL => no skip term
 *   z          (device) [batch, d_inner] dtype, NULL => no gate
 *   y          (device) [batch, d_inner] dtype, output
 *
 * Limits: 1 <= d_state <= 64.
 */
int mssm_state_update(float* state, const void* u, const void* delta, const float* A,
                      const void* Bm, const void* Cm, const float* Dskip, const void* z,
                      void* y, int64_t batch, int64_t d_inner, int64_t d_state,
                      mssm_dtype dtype, void* stream);

/*
 * Workspace (bytes) mssm_ssd_chunk_fwd needs for these sizes.  Host-only,
 * pure; returns 0 for invalid sizes.
 */
size_t mssm_ssd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                               int64_t headdim, int64_t d_state, int64_t ngroups,
                               int64_t chunk);

/*
 * Mamba-2 SSD, chunked.
 *
 * Defined by: "State-Space Model Optimization Patterns" page, section 2 "State Space Duality" --
 * Y(T,P) = SSM(A, B(T,N), C(T,N))(X(T,P)) with a scalar transition per
 * head, equivalently a structured masked attention; section 9 "Chunked
 * Computation" and section 2's algorithm -- split the sequence into chunks,
 * compute the chunk-local quadratic form and each chunk's final state, pass
 * states from chunk to chunk, combine; section 10 -- the mask is
 * semi-separable.  Mamba-2 layout from the "Mamba - Selective State Space Models" page ("Workflow 3":
 * d_state, headdim, ngroups).  The result equals, up to rounding, the
 * recurrence per (b, head h, head channel p) with head h using group
 * g = h / (nheads / ngroups):
 *
 *   H[n] <- exp(dt[b,t,h] * A[h]) * H[n] + dt[b,t,h] * x[b,t,h,p] * Bm[b,t,g,n]
 *   y[b,t,h,p] = (sum_n Cm[b,t,g,n] * H[n] + D[h] * x[b,t,h,p]) * silu(z[b,t,h,p])
 *
 *   x          (device) [batch, seqlen, nheads, headdim] dtype
 *   dt         (device) [batch, seqlen, nheads] dtype (positive; used as given)
 *   A          (device) [nheads] float32
 *   Bm, Cm     (device) [batch, seqlen, ngroups, d_state] dtype
 *   Dskip      (device) [nheads] float32, NULL => no skip term
 *   z          (device) [batch, seqlen, nheads, headdim] dtype, NULL => no gate
 *   h0         (device) [batch, nheads, headdim, d_state] float32, NULL => zero start
 *   y          (device) [batch, seqlen, nheads, headdim] dtype, output
 *   h_final    (device) [batch, nheads, headdim, d_state] float32, NULL => not written
 *   workspace  (device) scratch of at least mssm_ssd_workspace_size(...) bytes,
 *              owned by the caller; contents on entry are ignored and on exit
 *              are unspecified.  May be NULL if that size is 0.
 *
 * Limits: dtype MSSM_F32 or MSSM_BF16; headdim >= 1; 1 <= d_state <= 256;
 * chunk in {64, 128, 256}; nheads a multiple of ngroups; one batch row of
 * x, B and C below 2 GiB.  Other sizes return MSSM_ERR_UNSUPPORTED.  Any
 * seqlen >= 0 is accepted (a last partial chunk is handled).  The chunk is
 * the length of the blocks of the quadratic (attention-like) form; the
 * result does not depend on it beyond rounding.
 *
 * Two implementations, chosen from the arguments: bf16 with headdim a
 * multiple of 32 and d_state in {32, 64, 128, 256} runs on the bf16 matrix
 * cores with the chunk as given; every other call (float32 storage, other
 * headdims or d_state) runs on the fp32 matrix cores in chunks of 32 tokens.
 * The workspace holds the first's operand tiles, or the second's chunk
 * scores (none at d_state above 128); mssm_ssd_workspace_size reports a size
 * enough for whichever of the two the sizes lead to, whatever the dtype.
 */
int mssm_ssd_chunk_fwd(const void* x, const void* dt, const float* A, const void* Bm,
                       const void* Cm, const float* Dskip, const void* z, const float* h0,
                       void* y, float* h_final, int64_t batch, int64_t seqlen,
                       int64_t nheads, int64_t headdim, int64_t d_state, int64_t ngroups,
                       int64_t chunk, void* workspace, size_t workspace_bytes,
                       mssm_dtype dtype, void* stream);

/*
 * mssm_ssd_chunk_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace: its scratch is a fixed array of
 * MSSM_NOALLOC_SCRATCH_BYTES in device memory, one copy per GPU, which stays
 * reserved until the process ends.  Arguments, layouts, limits and results
 * are those of mssm_ssd_chunk_fwd; the caller still passes every input and
 * output.  Sizes whose workspace (mssm_ssd_workspace_size) exceeds the array
 * return MSSM_ERR_WORKSPACE, before anything is enqueued.  The call itself
 * allocates nothing; the first call on a device looks the array's address up
 * once (hipGetSymbolAddress).
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (the kernels write every scratch byte they read, so no clearing is
 * needed): calls that may overlap on one GPU -- on different streams, or from
 * different threads without ordering -- race on it and must not be issued.
 */
#define MSSM_NOALLOC_SCRATCH_BYTES (64LL << 20)
int mssm_ssd_chunk_fwd_noalloc(const void* x, const void* dt, const float* A, const void* Bm,
                               const void* Cm, const float* Dskip, const void* z,
                               const float* h0, void* y, float* h_final, int64_t batch,
                               int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t d_state, int64_t ngroups, int64_t chunk,
                               mssm_dtype dtype, void* stream);

/*
 * Mamba-2 decode: one token of the SSD recurrence, state updated in place.
 *
 * Defined by: "Mamba - Selective State Space Models" page, "Workflow 3" --
 * the Mamba-2 block (multi-head, headdim, d_state, ngroups); "State-Space
 * Model Optimization Patterns" page, section 2 -- a scalar transition per
 * head; "Mamba Architecture Details" page, "Hardware-Aware Implementation",
 * sequential mode -- a constant-size state updated per token, y read from
 * the UPDATED state.  For every (b, head h, head channel p), with group
 * g = h / (nheads / ngroups):
 *
 *   state[b,h,p,n] <- exp(dt[b,h] * A[h]) * state[b,h,p,n] + dt[b,h] * x[b,h,p] * Bm[b,g,n]
 *   y[b,h,p] = (sum_n Cm[b,g,n] * state[b,h,p,n] + D[h] * x[b,h,p]) * silu(z[b,h,p])
 *
 * It equals one token of mssm_ssd_chunk_fwd started from h0 = state.
 *
 *   state      (device) [batch, nheads, headdim, d_state] float32, read and overwritten
 *   x          (device) [batch, nheads, headdim] dtype
 *   dt         (device) [batch, nheads] dtype (positive; used as given)
 *   A          (device) [nheads] float32
 *   Bm, Cm     (device) [batch, ngroups, d_state] dtype
 *   Dskip      (device) [nheads] float32, NULL => no skip term
 *   z          (device) [batch, nheads, headdim] dtype, NULL => no gate
 *   y          (device) [batch, nheads, headdim] dtype, output
 *
 * Limits: 1 <= d_state <= 256 (MSSM_ERR_UNSUPPORTED otherwise; the sizes
 * mssm_ssd_chunk_fwd takes, so its h_final can seed decoding);
 * nheads % ngroups == 0 (MSSM_ERR_SHAPE).  batch, nheads or headdim = 0 is a
 * no-op.
 */
int mssm_ssd_state_update(float* state, const void* x, const void* dt, const float* A,
                          const void* Bm, const void* Cm, const float* Dskip, const void* z,
                          void* y, int64_t batch, int64_t nheads, int64_t headdim,
                          int64_t d_state, int64_t ngroups, mssm_dtype dtype, void* stream);

/* Message for the calling thread's last non-OK return ("" if none). */
const char* mssm_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int mssm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSSM_H */
