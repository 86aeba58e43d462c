/*
 * selscan.h -- C ABI of the MI355X (gfx950) S6 selective-scan library.
 *
 * Two operations, both defined on the Mamba pages:
 *
 *  selscan_fwd           the selective-scan forward over a whole sequence:
 *                        Delta_t = softplus(Delta_raw + bias), A_bar = exp(Delta_t A)
 *                        with diagonal A, B_bar u = Delta_t B_t u_t, the recurrence
 *                        h_t = A_bar_t * h_{t-1} + B_bar_t u_t, the readout
 *                        y_t = C_t . h_t + D u_t and the optional SiLU(z) gate.
 *                        Sources: Mamba tutorial (pwwt.cn) §2.2 (discretisation,
 *                        B_bar simplified to Delta B), §3.1 (B, C, Delta depend on
 *                        the input; softplus on Delta), §3.2 (one fused kernel,
 *                        parallel scan), §4.2 (the reference loop: h starts at 0,
 *                        readout after the update, + x D, then * SiLU(z));
 *                        Gu & Dao deep-reading report (zako-mio.github.io) §2.3,
 *                        §2.4 (the state h of shape (B,L,D,N) is never written
 *                        to HBM; only y of shape (B,L,D) is).
 *
 *  selscan_fwd_ex        the same forward with the variants the pages describe:
 *                        exact zero-order hold B_bar = (exp(Delta A) - 1) / A * B
 *                        (tutorial §2.2, selection-mechanism article discosf.com
 *                        §2.1), the reverse scan direction (the bidirectional use of
 *                        the tutorial's §7 outlook) and the causal depthwise
 *                        conv1d + SiLU that precedes the scan in the Mamba block
 *                        (tutorial §3.3 and its §4.2 listing), fused as a prologue.
 *
 *  selscan_bwd           gradients of selscan_fwd with respect to every input
 *                        (u, Delta_raw, A, B, C, D, z, the Delta bias and h0) for
 *                        an upstream gradient of y (and of h_last).  The states
 *                        are recomputed, not stored by the forward: Gu & Dao
 *                        deep-reading report §2.4 (recomputation in the backward
 *                        pass), selection-mechanism article (discosf.com) §3.4.
 *
 *  selscan_bwd_ex        gradients of selscan_fwd_ex (the variants above), and of
 *                        the conv prologue's taps and bias.
 *
 *  selscan_state_update  one decode step of the same recurrence on a resident
 *                        state: constant memory and O(1) work per token, one
 *                        state per sample.  Sources: Mamba tutorial §5.1 table
 *                        and §6.3; paper walkthrough (m.lqnn.cn) §3.2, which
 *                        names the single-token state update.
 *
 * Notation: the pages' B (batch) and D (channels) clash with the input matrix
 * B and the skip vector D, so the ABI calls them `batch` and `dim`, and the
 * matrices `Bm`, `Cm` and the skip vector `D_skip`.  N is the state size.
 *
 * Layout: every array is dense, row-major (C order), no strides:
 *   u, delta, z, y          (batch, L, dim)     element type = dtype
 *   Bm, Cm                  (batch, L, N)       element type = dtype
 *                           (B_t and C_t are shared by all dim channels)
 *   A                       (dim, N)            fp32 (diagonal A, one row per channel)
 *   D_skip, delta_bias      (dim)               fp32
 *   h0, h_last, state       (batch, dim, N)     fp32
 * For selscan_state_update the L axis is absent: u, delta, z, y are
 * (batch, dim) and Bm, Cm are (batch, N).
 *
 * dtype: SELSCAN_F32 or SELSCAN_BF16.  It applies to u, delta, Bm, Cm, z and y
 * together.  A, D_skip, delta_bias and the state are always fp32.  All
 * arithmetic is fp32; y is rounded to bf16 once, to nearest even.
 *
 * Pointers are device pointers (hipMalloc'd or equivalent), 16-byte aligned.
 * `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *
 * Ownership: the caller owns every buffer, the workspace included.  The library
 * keeps no state between calls.  It never allocates, frees or synchronises.
 * Inputs are only read.  Outputs must not overlap inputs; the exception is
 * `state`, which selscan_state_update updates in place.  Every buffer must stay
 * alive until the work queued on `stream` has completed.  Calls on different
 * streams may run concurrently if each has its own outputs and workspace.
 *
 * Errors: every argument check runs on the host, synchronously, BEFORE any
 * HIP call.  On an argument error the function returns a nonzero status,
 * queues nothing and touches no output.  SELSCAN_ERR_HIP means a HIP runtime
 * call (kernel launch) failed; selscan_last_hip_error() then returns the
 * hipError_t of the calling thread.  Otherwise the calls return SELSCAN_OK as
 * soon as the work is queued (asynchronous on `stream`).  NaN or Inf in the
 * inputs propagate to the outputs; there is no trap.
 */
#ifndef SELSCAN_H
#define SELSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SELSCAN_ABI_VERSION 8

enum selscan_dtype {
    SELSCAN_F32 = 0,
    SELSCAN_BF16 = 1
};

enum selscan_status {
    SELSCAN_OK = 0,
    SELSCAN_ERR_NULL = 1,        /* a required pointer is NULL                       */
    SELSCAN_ERR_SHAPE = 2,       /* a size is < 1, or an element count overflows     */
    SELSCAN_ERR_DTYPE = 3,       /* dtype is neither SELSCAN_F32 nor SELSCAN_BF16    */
    SELSCAN_ERR_UNSUPPORTED = 4, /* N not in the compiled set, dim > 2^24 (forward),
                                    a launch grid past 2^31 - 1 workgroups (see
                                    selscan_fwd), or a pointer that is not 16-byte
                                    aligned                                          */
    SELSCAN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required          */
    SELSCAN_ERR_ALIAS = 6,       /* an output buffer overlaps an input buffer        */
    SELSCAN_ERR_HIP = 7,         /* a HIP runtime call failed                        */
    SELSCAN_ERR_TIMEOUT = 8,     /* selscan_fwd_status: a bounded wait in a kernel
                                    gave up, the outputs of that call are invalid    */
    SELSCAN_ERR_TOO_LARGE = 9    /* selscan_fwd_noalloc: the shape needs more than
                                    SELSCAN_NOALLOC_SCRATCH_BYTES of workspace       */
};

/* SELSCAN_ABI_VERSION of the built library. */
int selscan_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *selscan_status_string(int status);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int selscan_last_hip_error(void);

/* Nonzero if N is a compiled state size (4, 8, 16, 32 and 64 are built). */
int selscan_supports_n(int64_t N);

/*
 * Completion status of the last selscan_fwd queued on `stream` with this
 * workspace.  Only the single-pass plan with decoupled look-back
 * (SELSCAN_FORCE_PLAN=lookback in the environment; the chunked scan with a
 * carry passed between blocks of the paper walkthrough (m.lqnn.cn) §3.2)
 * has waits between waves; each is bounded (SELSCAN_LOOKBACK_SPIN_LIMIT polls
 * if set, else about 2^20).  A wave whose wait gives up sets a status word
 * in the workspace and poisons its state with NaN, so its sequence part and
 * every later part of its channel group come out NaN.
 *
 * Under that plan this call waits for `stream`, reads the word and returns
 * SELSCAN_ERR_TIMEOUT if it is set, SELSCAN_OK otherwise (SELSCAN_ERR_HIP if
 * the read fails; SELSCAN_ERR_NULL for a NULL workspace).  Under any other
 * plan nothing can time out: it returns SELSCAN_OK at once, touching nothing.
 * Unlike the compute calls, it synchronises.
 */
int selscan_fwd_status(const void *workspace, void *stream);

/*
 * Bytes of device workspace selscan_fwd needs for this shape (0 is possible:
 * then `workspace` may be NULL).  Returns 0 for invalid arguments too; call
 * selscan_fwd to get the status.  The workspace holds per-chunk carries of
 * the sequence split.  Its contents need no initialisation, and its size
 * depends only on these arguments.
 */
size_t selscan_fwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N, int dtype);

/*
 * Selective-scan forward.
 *
 *   u          (batch, L, dim)  dtype   input sequence u_t (x in the pages)
 *   delta      (batch, L, dim)  dtype   Delta_raw, before bias and softplus
 *   A          (dim, N)         fp32    diagonal state matrix (negative for decay)
 *   Bm, Cm     (batch, L, N)    dtype   input-dependent B_t and C_t
 *   D_skip     (dim)            fp32    skip term D; NULL means 0
 *   z          (batch, L, dim)  dtype   gate input; NULL means no gate
 *   delta_bias (dim)            fp32    added to Delta_raw; NULL means 0
 *   delta_softplus  1: Delta_t = softplus(Delta_raw + bias); 0: Delta_raw + bias
 *   h0         (batch, dim, N)  fp32    initial state; NULL means zeros
 *   y          (batch, L, dim)  dtype   output, written
 *   h_last     (batch, dim, N)  fp32    final state h_L, written; NULL to skip
 *   workspace / workspace_bytes         >= selscan_fwd_workspace_bytes(...)
 *   stream                              hipStream_t as void*
 *
 * Required: batch, L, dim >= 1; dim <= 2^24; N supported; u, delta, A, Bm, Cm,
 * y non-NULL; batch * ceil(dim/64) * max(ceil(L/16), N) < 2^31 (every launch
 * grid fits; far beyond any shape whose arrays fit in device memory).  The
 * workspace-size functions return 0 for shapes that violate these.
 *
 * Plans: the default is the two-pass streaming scan.  The environment
 * variable SELSCAN_FORCE_PLAN selects an ablation with the same results
 * within the tolerances: lookback (single pass with decoupled look-back),
 * chunked (segments of a chunk joined through LDS) or dpp (the lanes of a
 * wave hold 64 steps of one channel, scanned with DPP; one wave per channel,
 * so batch * dim * parts / 4 must stay below 2^31 workgroups, else
 * SELSCAN_ERR_HIP).  The workspace size covers every plan.
 */
int selscan_fwd(const void *u, const void *delta, const float *A,
                const void *Bm, const void *Cm, const float *D_skip,
                const void *z, const float *delta_bias, int delta_softplus,
                const float *h0, void *y, float *h_last,
                int64_t batch, int64_t L, int64_t dim, int64_t N, int dtype,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * forward of selscan_fwd without a workspace argument.  Its workspace is a
 * fixed device array inside the library, SELSCAN_NOALLOC_SCRATCH_BYTES
 * (128 MiB) on every device the library runs on, held until the process
 * ends.  The call allocates and frees nothing: on its first call on a device
 * it looks up that device's copy of the array (hipGetSymbolAddress, with
 * that device current), later calls reuse the address.
 *
 * Arguments, results and errors as selscan_fwd (the same kernels and plan,
 * so the same y and h_last bit for bit), without workspace and
 * workspace_bytes, plus SELSCAN_ERR_TOO_LARGE when
 * selscan_fwd_workspace_bytes(batch, L, dim, N, dtype) exceeds
 * SELSCAN_NOALLOC_SCRATCH_BYTES (the workloads here need at most about
 * 83 MiB at N = 16: batch 16 x L 2048 x dim 5120, or L 131072 x dim 2048),
 * detected on the host before any HIP call.  The array needs no clearing
 * between calls (every call writes what it later reads).
 *
 * All calls on one device share that device's array: two calls that may
 * overlap in time on one device (different streams, or host threads with
 * no ordering between their streams) race on it and may return wrong
 * results.  Calls on one stream are ordered and safe.
 */
#define SELSCAN_NOALLOC_SCRATCH_BYTES (128u << 20)
int selscan_fwd_noalloc(const void *u, const void *delta, const float *A,
                        const void *Bm, const void *Cm, const float *D_skip,
                        const void *z, const float *delta_bias, int delta_softplus,
                        const float *h0, void *y, float *h_last,
                        int64_t batch, int64_t L, int64_t dim, int64_t N, int dtype,
                        void *stream);

/* Flags of selscan_fwd_ex. */
#define SELSCAN_FLAG_ZOH_EXACT 1   /* B_bar = (exp(Delta A) - 1) / A * B, Delta B where A = 0 */
#define SELSCAN_FLAG_REVERSE   2   /* scan from t = L-1 down to t = 0                      */
#define SELSCAN_FLAG_REUSE_FWD_STATE 4   /* selscan_bwd_ex only: see there                 */
#define SELSCAN_FLAG_KEEP_CHECKPOINTS 8  /* selscan_fwd_ex, then selscan_bwd_ex: see there */
#define SELSCAN_MAX_CONV_WIDTH 4

/*
 * Selective-scan forward with variants.  Arguments as selscan_fwd, plus:
 *
 *   flags        0 or an OR of SELSCAN_FLAG_ZOH_EXACT, SELSCAN_FLAG_REVERSE; or
 *                SELSCAN_FLAG_KEEP_CHECKPOINTS, alone or with REVERSE (below).
 *                ZOH_EXACT: the state update is
 *                  h = exp(Delta A) h + (exp(Delta A) - 1) / A * B u
 *                instead of h = exp(Delta A) h + Delta B u (the limit Delta B u
 *                where A[d,n] = 0).
 *                REVERSE: the whole computation runs on the time-reversed
 *                sequence and y is returned in the original order: the
 *                recurrence is h_t = A_bar_t h_{t+1} + B_bar_t u_t from t = L-1
 *                down to 0, h0 is the state entering t = L-1 and h_last the
 *                state after t = 0.  The conv prologue is then causal in the
 *                reversed time (its taps reach t+1 .. t+k-1).
 *   conv_weight  (dim, conv_width) fp32, depthwise causal conv taps; used when
 *                conv_width > 0, and then required.
 *   conv_bias    (dim) fp32 or NULL (0).
 *   conv_width   0: no prologue, u is the scan input (conv_weight and conv_bias
 *                are ignored).  1..SELSCAN_MAX_CONV_WIDTH: the scan input is
 *                  u'[b,t,d] = SiLU(conv_bias[d] + sum_j conv_weight[d,j] *
 *                                   u[b, t-(conv_width-1)+j, d])
 *                with u = 0 before t = 0, and D u in the readout uses u'.
 *
 * With flags = 0 and conv_width = 0 this is the default forward itself (the
 * results of selscan_fwd bit for bit).
 *
 * SELSCAN_FLAG_KEEP_CHECKPOINTS (alone or with REVERSE: with ZOH_EXACT or
 * conv_width > 0, SELSCAN_ERR_UNSUPPORTED): the forward of a training step
 * whose backward reuses this workspace (selscan_bwd_ex with
 * SELSCAN_FLAG_REUSE_FWD_STATE | SELSCAN_FLAG_KEEP_CHECKPOINTS and the same
 * REVERSE flag).  The main pass also stores the state entering every 4-step
 * chunk of the scan, the checkpoints
 * that backward's recomputation would otherwise walk the sequence for: 4 N
 * bytes per element (the paper walkthrough (m.lqnn.cn) §5.4: with memory to
 * spare, recompute less).  The workspace must then hold
 * selscan_bwd_workspace_bytes (SELSCAN_ERR_WORKSPACE otherwise).  y and
 * h_last are bit for bit those of the call without the flag.
 *
 * Workspace: the same size as selscan_fwd (selscan_fwd_workspace_bytes).
 * Errors as selscan_fwd, and: SELSCAN_ERR_UNSUPPORTED for an unknown flag bit
 * or conv_width > SELSCAN_MAX_CONV_WIDTH, SELSCAN_ERR_SHAPE for conv_width < 0,
 * SELSCAN_ERR_NULL for conv_width > 0 without conv_weight.  conv_weight and
 * conv_bias are inputs: they must not overlap y or h_last.
 * The SELSCAN_FORCE_PLAN ablation does not apply to this call.
 */
int selscan_fwd_ex(const void *u, const void *delta, const float *A,
                   const void *Bm, const void *Cm, const float *D_skip,
                   const void *z, const float *delta_bias, int delta_softplus,
                   const float *h0, void *y, float *h_last,
                   int64_t batch, int64_t L, int64_t dim, int64_t N, int dtype,
                   int flags, const float *conv_weight, const float *conv_bias,
                   int64_t conv_width,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace selscan_bwd needs for this shape (never 0 for a
 * valid shape; 0 for invalid arguments).  It holds the part summaries of the
 * forward and of the adjoint, the recomputation checkpoints (the state at the
 * start of every 4-step chunk: batch * ceil(dim/64) * ceil(L/4) * N * 256
 * bytes), the partial sums of the reduced gradients and, for the conv
 * prologue of selscan_bwd_ex, its output and that output's gradient (fp32,
 * batch * L * dim * 4 bytes, counted for every call: the size takes no
 * flags).  No initialisation.  The same size serves selscan_bwd_ex, with or
 * without the conv prologue.
 */
size_t selscan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N, int dtype);

/*
 * Backward of selscan_fwd (B_bar = Delta B, forward direction).  With
 * ypre_t = C_t.h_t + D u_t, y_t = ypre_t SiLU(z_t), dypre_t = dy_t SiLU(z_t)
 * and the adjoint lambda_t = C_t dypre_t + exp(Delta_{t+1} A) lambda_{t+1}
 * (plus dh_last at t = L-1), it returns the gradient of
 *     sum(dy * y) + sum(dh_last * h_last)
 * with respect to each input:
 *   du[b,t,d]      = dypre D[d] + Delta sum_n lambda[n] B_t[n]
 *   ddelta[b,t,d]  = dDelta * sigmoid(Delta_raw + bias)  (dDelta with softplus off),
 *                    dDelta = sum_n lambda[n] (A[d,n] A_bar[n] h_{t-1}[n] + B_t[n] u)
 *   dA[d,n]        = sum_{b,t} lambda[n] Delta A_bar[n] h_{t-1}[n]
 *   dB[b,t,n]      = sum_d lambda[n] Delta u        dC[b,t,n] = sum_d dypre h_t[n]
 *   dD[d]          = sum_{b,t} dypre u              ddelta_bias[d] = sum_{b,t} ddelta
 *   dz[b,t,d]      = dy ypre SiLU'(z)               dh0[b,d,n] = A_bar_0[n] lambda_0[n]
 *
 *   inputs        as selscan_fwd (u, delta, A, Bm, Cm, D_skip, z, delta_bias,
 *                 delta_softplus, h0), and
 *   dy            (batch, L, dim)  dtype   upstream gradient of y
 *   dh_last       (batch, dim, N)  fp32    upstream gradient of h_last; NULL = 0
 *   du, ddelta    (batch, L, dim)  dtype   written
 *   dz            (batch, L, dim)  dtype   written; required when z is given,
 *                                          ignored when z is NULL
 *   dA            (dim, N)         fp32    written
 *   dB, dC        (batch, L, N)    fp32    written
 *   dD, ddelta_bias (dim)          fp32    written; NULL to skip (defined even
 *                                          when D_skip / delta_bias are NULL)
 *   dh0           (batch, dim, N)  fp32    written; NULL to skip
 *   workspace     >= selscan_bwd_workspace_bytes(...), 16-byte aligned
 *
 * dB, dC, dA, dD and ddelta_bias are sums in a fixed order (bitwise
 * repeatable).  Errors as selscan_fwd; every output must be disjoint from
 * every input and from the other outputs (SELSCAN_ERR_ALIAS).
 */
int selscan_bwd(const void *u, const void *delta, const float *A,
                const void *Bm, const void *Cm, const float *D_skip,
                const void *z, const float *delta_bias, int delta_softplus,
                const float *h0, const void *dy, const float *dh_last,
                void *du, void *ddelta, float *dA, float *dB, float *dC,
                float *dD, void *dz, float *ddelta_bias, float *dh0,
                int64_t batch, int64_t L, int64_t dim, int64_t N, int dtype,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward of selscan_fwd_ex: the gradient of
 *     sum(dy * y) + sum(dh_last * h_last)
 * for the forward that selscan_fwd_ex computes with the same flags and conv
 * prologue.  Arguments as selscan_bwd, plus flags, conv_weight, conv_bias and
 * conv_width as selscan_fwd_ex, and:
 *   dconv_weight  (dim, conv_width) fp32  written; required when conv_width > 0
 *   dconv_bias    (dim)             fp32  written; NULL to skip (defined even
 *                                         when conv_bias is NULL)
 * Both are ignored when conv_width = 0.  With the conv prologue, du is the
 * gradient of the raw input u (the conv's input).  With REVERSE, h0 and dh0
 * belong to the state entering t = L-1, dh_last to the state after t = 0.
 * With ZOH_EXACT, the B_bar coefficient c = (exp(Delta A) - 1) / A replaces
 * Delta in du, dB and the dDelta, dA terms of B_bar: dc/dDelta = exp(Delta A),
 * dc/dA = (Delta exp(Delta A) - c) / A (Delta^2 / 2 where A = 0).
 * Sources: as selscan_fwd_ex for the forward; the gradients are its exact
 * derivatives (the recomputation as for selscan_bwd).
 *
 * Workspace: selscan_bwd_workspace_bytes.  dconv_weight and dconv_bias are
 * sums in a fixed order (bitwise repeatable) like dA.  Errors as selscan_bwd
 * and selscan_fwd_ex, and SELSCAN_ERR_NULL for conv_width > 0 without
 * dconv_weight.
 *
 * SELSCAN_FLAG_REUSE_FWD_STATE (in flags, with REVERSE or alone; not with
 * ZOH_EXACT or conv_width > 0, SELSCAN_ERR_UNSUPPORTED): the workspace is the
 * one the matching forward last ran in (selscan_fwd, or selscan_fwd_ex with
 * the same REVERSE flag and no other variant, under the default plan: with
 * SELSCAN_FORCE_PLAN set to another plan the flag is SELSCAN_ERR_UNSUPPORTED,
 * since that forward leaves another layout) with the same u, delta, A, Bm,
 * delta_bias, delta_softplus, h0 and sizes, and still holds that forward's
 * sequence-part summaries and part entry states, which the backward then
 * reads instead of recomputing (the forward's summary and carry passes).
 * The result is bit for bit that of the call without the flag.  The library
 * cannot check the correspondence: it is the caller's to keep.  A workspace
 * of selscan_bwd_workspace_bytes is large enough for the forward too.
 *
 * SELSCAN_FLAG_KEEP_CHECKPOINTS (with SELSCAN_FLAG_REUSE_FWD_STATE, so plain
 * or with REVERSE alone; SELSCAN_ERR_UNSUPPORTED without the reuse): that
 * forward was run with SELSCAN_FLAG_KEEP_CHECKPOINTS as well, and the
 * workspace also holds its checkpoint states; the backward reads them and
 * skips its own checkpoint pass (and the forward entry states it needs).
 * The gradients are within rounding of the call without the flag (the
 * forward's states where the checkpoint pass would recompute them).
 */
int selscan_bwd_ex(const void *u, const void *delta, const float *A,
                   const void *Bm, const void *Cm, const float *D_skip,
                   const void *z, const float *delta_bias, int delta_softplus,
                   const float *h0, const void *dy, const float *dh_last,
                   void *du, void *ddelta, float *dA, float *dB, float *dC,
                   float *dD, void *dz, float *ddelta_bias, float *dh0,
                   int flags, const float *conv_weight, const float *conv_bias,
                   int64_t conv_width, float *dconv_weight, float *dconv_bias,
                   int64_t batch, int64_t L, int64_t dim, int64_t N, int dtype,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step, updating `state` in place:
 *   state[b,d,n] <- exp(Delta A[d,n]) * state[b,d,n] + Delta Bm[b,n] u[b,d]
 *   y[b,d]        = (sum_n Cm[b,n] state[b,d,n] + D[d] u[b,d]) * SiLU(z[b,d])
 * with Delta = softplus(delta[b,d] + bias[d]) (or the raw sum), exactly one
 * t-step of selscan_fwd.
 *
 *   state      (batch, dim, N)  fp32    read and written in place
 *   u, delta   (batch, dim)     dtype
 *   A          (dim, N)         fp32
 *   Bm, Cm     (batch, N)       dtype
 *   D_skip, delta_bias (dim)    fp32    NULL means 0
 *   z          (batch, dim)     dtype   NULL means no gate
 *   y          (batch, dim)     dtype   output, written
 *
 * Required: batch, dim >= 1; N supported; batch * dim * N < 2^31 (the state
 * is indexed with 32 bits: SELSCAN_ERR_UNSUPPORTED beyond); state, u, delta,
 * A, Bm, Cm, y non-NULL.
 */
int selscan_state_update(float *state, const void *u, const void *delta, const float *A,
                         const void *Bm, const void *Cm, const float *D_skip,
                         const void *z, const float *delta_bias, int delta_softplus,
                         void *y, int64_t batch, int64_t dim, int64_t N, int dtype,
                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SELSCAN_H */
