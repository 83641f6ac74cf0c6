/*
 * ss_scan.h -- C ABI of the MI355X (gfx950) selective-scan library
 * (libss_scan.so).
 *
 * The library computes the Mamba selective scan with a softplus step size and
 * its single-token state-update (decode) step, entirely in HIP kernels.  The
 * operation is the one defined by
 *   - mhpn.cn, "PyTorch新手也能懂：手把手拆解Mamba-minimal中的selective_scan实现":
 *     section 2 (argument shapes), sections 3, 3.1, 3.2 (exp(delta*A) for A,
 *     delta*B*u for B), section 4 (sequential recurrence from a zero state,
 *     readout with C after each update), section 5 (y += u*D), section 7
 *     (A = -exp(A_log), softplus keeps delta positive);
 *   - jiafeimiao.top, "代码连连看——mamba", the Mamba.step listing and the
 *     selective_state_update call that follows it (bias added to dt inside the
 *     softplus, in-place state update, gate y * silu(z) after the D skip),
 *     and the convolution step that comes before it (ss_conv_update).
 *
 * For every batch b, channel d and time t (h starts at zero, or at a given
 * initial state with the _ex entry points):
 *     delta' = softplus(delta[b,t,d] + bias[d])      (or delta + bias without softplus)
 *     h[k]   = exp(delta' * A[d,k]) * h[k] + delta' * B[b,t,k] * u[b,t,d],  A = -exp(A_log)
 *     y      = sum_k C[b,t,k] * h[k] + D[d] * u[b,t,d]
 *     y      = y * z / (1 + exp(-z))                  (only when z is given)
 * The _ex entry points can instead weight the input term with the zero-order
 * hold (mhpn.cn page, section 6: the exact discretisation of the B term, which
 * the simplified delta' * B above approximates; A is diagonal, so it acts per
 * state):
 *     h[k]   = exp(delta' * A[d,k]) * h[k] + (exp(delta' * A[d,k]) - 1) / A[d,k] * B[b,t,k] * u[b,t,d]
 *
 * Conventions shared by every entry point:
 *   - Every pointer is DEVICE memory owned by the caller.  Tensors are dense,
 *     contiguous and row-major (last index fastest) with the shapes stated.
 *   - u, delta, B, C, z and y (x, dt of the step) share one element type,
 *     `dtype` (SS_F32 or SS_BF16).  A_log, D, the bias and the state are
 *     always fp32.  bf16 results are rounded to nearest even.
 *   - Nothing is allocated, no pointer is kept after return, and there is no
 *     hidden global state apart from a per-device cache of attributes, so
 *     calls from several host threads are safe.  Calls that share a
 *     workspace must not overlap.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and runs asynchronously; results are valid once the stream
 *     has been synchronised.  The library never synchronises.
 *   - Arguments are validated before anything is enqueued; on any error
 *     nothing is launched and nothing is written.
 *   - Outputs must not overlap any input (SS_ERR_ALIAS); the state of the
 *     step is the one in/out buffer and is updated in place, and the
 *     initial_state of ss_scan_fwd_ex may be its last_state buffer itself.
 *   - Pointers must be aligned to their element size (SS_ERR_ALIGN), and
 *     workspaces to 256 bytes.
 *   - A long scan is cut into segments along L that hand the state on
 *     through the workspace; a segment waits (bounded) for its predecessor.
 *     Such a wait cannot deadlock, but should one give up, the scan goes on
 *     from NaN and records it: ss_scan_status then reports SS_ERR_TIMEOUT.
 */
#ifndef SS_SCAN_H
#define SS_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of u, delta, B, C, z, y (and x, dt of the step). */
typedef enum {
    SS_F32 = 0,
    SS_BF16 = 1
} ss_dtype;

/* Return codes. */
typedef enum {
    SS_OK = 0,
    SS_ERR_NULL = -1,        /* a required pointer is NULL                          */
    SS_ERR_SHAPE = -2,       /* a size is <= 0, or too large to index or above SS_MAX_CHANNELS */
    SS_ERR_DTYPE = -3,       /* dtype is not an ss_dtype value                      */
    SS_ERR_UNSUPPORTED = -4, /* n (the state size) is above SS_MAX_STATE            */
    SS_ERR_WORKSPACE = -5,   /* workspace missing or smaller than the query says    */
    SS_ERR_HIP = -6,         /* the HIP runtime refused the launch                  */
    SS_ERR_ALIAS = -7,       /* an output overlaps an input                         */
    SS_ERR_ALIGN = -8,       /* a pointer is not aligned to its element size        */
    SS_ERR_MODE = -9,        /* discretization is not an ss_discretization value    */
    SS_ERR_TIMEOUT = -10     /* (ss_scan_status) a wait between segments gave up    */
} ss_status;

/* Input term of the recurrence (the _ex entry points). */
typedef enum {
    SS_DISC_EULER = 0,       /* delta' * B * u, as ss_scan_fwd and ss_state_update  */
    SS_DISC_ZOH = 1          /* (exp(delta' * A) - 1) / A * B * u, the zero-order hold */
} ss_discretization;

/* How ss_cross_scan_fwd_ex merges the four directions of a map. */
typedef enum {
    SS_CROSS_AUTO = 0,       /* the library's choice: the two-pass form              */
    SS_CROSS_ONE_PASS = 1,   /* one kernel, the directions summed in LDS (n <= 4)    */
    SS_CROSS_TWO_PASS = 2    /* per-direction outputs in the workspace, then a merge  */
} ss_cross_form;

/* Largest state size n the kernels are built for. */
#define SS_MAX_STATE 64

/* Largest channel count d_in of ss_scan_fwd (per-thread offsets are 24-bit products). */
#define SS_MAX_CHANNELS ((1 << 24) - 1)

/*
 * Bytes of device workspace ss_scan_fwd needs for these sizes (0 when none).
 * The value depends only on the arguments, not on the device.  Returns 0 for
 * invalid arguments as well; ss_scan_fwd reports those.
 */
size_t ss_scan_fwd_workspace_bytes(int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype);

/*
 * Selective scan, forward (mhpn.cn page, sections 2-5; jiafeimiao.top page,
 * the softplus(dt + dt_bias) of Mamba.step).
 *
 *   u, delta   : (b, L, d_in)  dtype
 *   A_log      : (d_in, n)     fp32; the kernels use A = -exp(A_log).
 *                A caller holding A (all entries < 0) passes log(-A).
 *   B, C       : (b, L, n)     dtype; shared by all d_in channels
 *   D          : (d_in)        fp32, required (pass zeros for no skip)
 *   z          : (b, L, d_in)  dtype, or NULL for no gate
 *   delta_bias : (d_in)        fp32, or NULL for no bias
 *   delta_softplus : nonzero -> delta' = softplus(delta + bias); zero -> delta + bias
 *   y          : (b, L, d_in)  dtype, output
 *   last_state : (b, d_in, n)  fp32, output h after the last step, or NULL
 *   workspace  : device memory of at least ss_scan_fwd_workspace_bytes()
 *                bytes, 256-byte aligned (SS_ERR_ALIGN otherwise).  Its
 *                contents need no initialisation; after the call it holds
 *                the call's status (ss_scan_status) and scratch.
 * Any n in 1..SS_MAX_STATE, d_in in 1..SS_MAX_CHANNELS and b, L >= 1 with
 * b * L * d_in <= 2^46, L < 2^31 - 1024 and b * ceil(d_in / 64) < 2^22 are
 * accepted (no tile multiples are required); other sizes give SS_ERR_SHAPE.
 * Returns an ss_status.
 */
int ss_scan_fwd(const void *u, const void *delta, const float *A_log,
                const void *B, const void *C, const float *D,
                const void *z, const float *delta_bias, int delta_softplus,
                void *y, float *last_state,
                int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * ss_scan_fwd with two more inputs (mhpn.cn page: section 4 starts the
 * recurrence from a zero state, section 6 gives the zero-order hold):
 *
 *   initial_state  : (b, d_in, n) fp32, the state before the first step, or
 *                    NULL for zero.  It may be the same buffer as last_state
 *                    (the state is then carried over in place); any other
 *                    overlap with an output gives SS_ERR_ALIAS.
 *   discretization : an ss_discretization value (else SS_ERR_MODE).
 * Splitting a sequence into consecutive parts and passing each part's
 * last_state as the next part's initial_state gives the outputs of one scan
 * over the whole sequence (up to rounding).  All other arguments, sizes and
 * errors are those of ss_scan_fwd, which is this call with NULL and
 * SS_DISC_EULER.  Returns an ss_status.
 */
int ss_scan_fwd_ex(const void *u, const void *delta, const float *A_log,
                   const void *B, const void *C, const float *D,
                   const void *z, const float *delta_bias, int delta_softplus,
                   const float *initial_state, int discretization,
                   void *y, float *last_state,
                   int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Status a scan call left in its workspace, copied on `stream` (after that
 * call, in stream order) to *status, one int32 in device memory (or host
 * memory the device can write): SS_OK, or SS_ERR_TIMEOUT when a wait between
 * segments of L gave up, in which case the outputs of that call hold NaN.
 * workspace is the workspace passed to ss_scan_fwd(_ex), ss_cross_scan_fwd(_ex)
 * or ss_scan_bwd(_ex); NULL reads the static scratch of the last
 * ss_scan_fwd_noalloc call on the current device.  Returns an ss_status.
 */
int ss_scan_status(const void *workspace, size_t workspace_bytes, int32_t *status, void *stream);

/* Size of the static device array that ss_scan_fwd_noalloc works in. */
#define SS_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * ss_scan_fwd_ex without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The scratch is a static device array of
 * SS_NOALLOC_SCRATCH_BYTES bytes, one per device, looked up on the first call
 * on a device and held until the process ends; nothing is allocated or freed.
 * Where the segments along L that ss_scan_fwd_ex would use need more than
 * that, fewer segments are used (the results are the same, bit for bit;
 * only the speed differs), so every size ss_scan_fwd_ex accepts is accepted.
 * All calls on one device share the array: calls that overlap in time on
 * one device (several streams or host threads) race and must be avoided.
 * Arguments, sizes and errors otherwise as for ss_scan_fwd_ex.
 * Returns an ss_status.
 */
int ss_scan_fwd_noalloc(const void *u, const void *delta, const float *A_log,
                        const void *B, const void *C, const float *D,
                        const void *z, const float *delta_bias, int delta_softplus,
                        const float *initial_state, int discretization,
                        void *y, float *last_state,
                        int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype,
                        void *stream);

/*
 * One decode step on a persistent state (jiafeimiao.top page: Mamba.step and
 * its selective_state_update(ssm_state, x, dt, A, B, C, D, z, dt_bias,
 * dt_softplus) call; the state is updated in place).
 *
 *   state   : (b, d_in, n) fp32, read and overwritten with the new state
 *   x, dt   : (b, d_in)    dtype (dt is the value before bias and softplus)
 *   A_log   : (d_in, n)    fp32
 *   B, C    : (b, n)       dtype
 *   D       : (d_in)       fp32, required
 *   z       : (b, d_in)    dtype, or NULL for no gate
 *   dt_bias : (d_in)       fp32, or NULL
 *   dt_softplus : as delta_softplus above
 *   y       : (b, d_in)    dtype, output
 * Sizes: b, d_in >= 1, b * d_in < 2^28, b * d_in * n <= 2^46.
 * Returns an ss_status.
 */
int ss_state_update(float *state, const void *x, const void *dt,
                    const float *A_log, const void *B, const void *C,
                    const float *D, const void *z, const float *dt_bias,
                    int dt_softplus, void *y,
                    int64_t b, int64_t d_in, int64_t n, int dtype, void *stream);

/*
 * ss_state_update with the input term chosen by `discretization` (an
 * ss_discretization value, else SS_ERR_MODE; mhpn.cn page, section 6).  The
 * zero-order-hold step is one step of ss_scan_fwd_ex with SS_DISC_ZOH.  All
 * other arguments, sizes and errors are those of ss_state_update, which is
 * this call with SS_DISC_EULER.  Returns an ss_status.
 */
int ss_state_update_ex(float *state, const void *x, const void *dt,
                       const float *A_log, const void *B, const void *C,
                       const float *D, const void *z, const float *dt_bias,
                       int dt_softplus, int discretization, void *y,
                       int64_t b, int64_t d_in, int64_t n, int dtype, void *stream);

/*
 * VMamba's cross scan, fused (githubissues.com VMamba issue 206: CrossScan and
 * CrossMerge only arrange the sequence around the selective scan).  Each
 * H x W feature map is read as four sequences of L = H * W steps --
 * direction 0 row-major (step t = h*W + w), 1 column-major (t = w*H + h),
 * 2 and 3 the same two orders backwards -- each scanned as ss_scan_fwd scans
 * one batch row (zero initial state, delta' B u input term, no gate), and the
 * four outputs are added back at the positions they came from:
 *     y[m, p, d] = sum_k y_k[m, t_k(p), d]
 * The map is read in place by every direction (no unrolled copies); the
 * four outputs go to workspace and a second kernel adds them back, in the
 * order k = 0, 1, 2, 3, so y is the same bit for bit on every run.  This is
 * ss_cross_scan_fwd_ex with SS_CROSS_AUTO.
 *
 *   x          : (maps, H, W, d_in)    dtype; u of all four directions
 *   delta      : (maps, 4, L, d_in)    dtype; direction k's values in its own step order
 *   A_log      : (4, d_in, n)          fp32, one set per direction
 *   B, C       : (maps, 4, L, n)       dtype
 *   D          : (4, d_in)             fp32
 *   delta_bias : (4, d_in)             fp32, or NULL
 *   delta_softplus : as for ss_scan_fwd
 *   y          : (maps, H, W, d_in)    fp32 output (whatever dtype the inputs have)
 *   last_state : (maps, 4, d_in, n)    fp32 output, or NULL
 *   workspace  : device memory of ss_cross_scan_fwd_workspace_bytes() bytes,
 *                256-byte aligned (SS_ERR_ALIGN otherwise); it holds the four
 *                directions' outputs, 16 * maps * L * d_in bytes, and the
 *                scan's own workspace.
 * Sizes: those of ss_scan_fwd with b = 4 * maps and L = H * W.  Errors as
 * for ss_scan_fwd.
 */
size_t ss_cross_scan_fwd_workspace_bytes(int64_t maps, int64_t H, int64_t W,
                                         int64_t d_in, int64_t n, int dtype);

int ss_cross_scan_fwd(const void *x, const void *delta, const float *A_log,
                      const void *B, const void *C, const float *D,
                      const float *delta_bias, int delta_softplus,
                      float *y, float *last_state,
                      int64_t maps, int64_t H, int64_t W, int64_t d_in, int64_t n,
                      int dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ss_cross_scan_fwd with the merge chosen by `form` (an ss_cross_form value,
 * else SS_ERR_MODE):
 *   SS_CROSS_TWO_PASS (and SS_CROSS_AUTO): as ss_cross_scan_fwd.
 *   SS_CROSS_ONE_PASS: one kernel scans the four directions of a map and 8
 *     channels together and adds their outputs into that map slice's sum in
 *     LDS, writing y once; the per-direction outputs never reach memory
 *     (about 2.3x fewer bytes moved).  Each position takes its four terms in
 *     the order of the 64-step chunks in which they were formed, direction
 *     order within a chunk, so y is the same bit for bit on every run (and
 *     within fp32 rounding of the two-pass form).  It takes n <= 4 and maps
 *     whose sum fits in LDS, L = H * W up to 4265 at n = 1, 4205 at n = 2
 *     and 4084 at n = 3 and 4; other shapes return SS_ERR_UNSUPPORTED.
 * The workspace is ss_cross_scan_fwd_ex_workspace_bytes(..., form) bytes
 * (256 for the one-pass form: its status words), 256-byte aligned.  Other
 * arguments, sizes and errors as for ss_cross_scan_fwd.
 */
size_t ss_cross_scan_fwd_ex_workspace_bytes(int64_t maps, int64_t H, int64_t W,
                                            int64_t d_in, int64_t n, int dtype, int form);

int ss_cross_scan_fwd_ex(const void *x, const void *delta, const float *A_log,
                         const void *B, const void *C, const float *D,
                         const float *delta_bias, int delta_softplus,
                         float *y, float *last_state,
                         int64_t maps, int64_t H, int64_t W, int64_t d_in, int64_t n,
                         int dtype, int form, void *workspace, size_t workspace_bytes, void *stream);

/* Largest state size n of ss_scan_bwd. */
#define SS_MAX_BWD_STATE 64

/* Bytes of device workspace ss_scan_bwd needs (0 for invalid arguments). */
size_t ss_scan_bwd_workspace_bytes(int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype);

/*
 * Gradient of ss_scan_fwd_ex with the delta' * B * u input term (the pages
 * only name the autograd wrappers of the scan; the formulas are the chain
 * rule of the forward definition above).  Given the forward's inputs and
 * the gradients dy of y and dlast_state of last_state, writes the gradients
 * of every input:
 *   dy          : (b, L, d_in) dtype
 *   dlast_state : (b, d_in, n) fp32, or NULL (zero)
 *   du, ddelta  : (b, L, d_in) dtype      ddelta is with respect to delta before bias and softplus
 *   dA_log      : (d_in, n)    fp32       dB, dC : (b, L, n) dtype
 *   dD          : (d_in)       fp32       dz : (b, L, d_in) dtype, required when z is given
 *   ddelta_bias : (d_in) fp32, or NULL (only written when delta_bias is given)
 *   dinitial_state : (b, d_in, n) fp32, or NULL
 * The call runs the forward scan again (saving the state every 8 steps in
 * the workspace) and then the adjoint backwards in time; sums over channels,
 * batch rows and time are formed from per-workgroup partials in a fixed
 * order, so the results are the same bit for bit on every run.  Sizes as for
 * ss_scan_fwd with n <= SS_MAX_BWD_STATE (else SS_ERR_UNSUPPORTED); the
 * workspace must be 256-byte aligned and ss_scan_bwd_workspace_bytes() long.
 * No output may overlap an input, another output or the workspace
 * (SS_ERR_ALIAS).  Returns an ss_status.
 */
int ss_scan_bwd(const void *u, const void *delta, const float *A_log,
                const void *B, const void *C, const float *D,
                const void *z, const float *delta_bias, int delta_softplus,
                const float *initial_state, const void *dy, const float *dlast_state,
                void *du, void *ddelta, float *dA_log, void *dB, void *dC,
                float *dD, void *dz, float *ddelta_bias, float *dinitial_state,
                int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * ss_scan_bwd for either input term of ss_scan_fwd_ex: discretization is
 * SS_DISC_EULER (the same as ss_scan_bwd) or SS_DISC_ZOH, the gradient of the
 * zero-order-hold scan with input weight beta = (exp(delta' A) - 1) / A
 * (mhpn.cn page, section 6), whose derivatives are exp(delta' A) in delta'
 * and (delta' exp(delta' A) - beta) / A in A.  Arguments, workspace and
 * results otherwise as for ss_scan_bwd; another discretization value is
 * SS_ERR_MODE.
 */
int ss_scan_bwd_ex(const void *u, const void *delta, const float *A_log,
                   const void *B, const void *C, const float *D,
                   const void *z, const float *delta_bias, int delta_softplus,
                   const float *initial_state, int discretization,
                   const void *dy, const float *dlast_state,
                   void *du, void *ddelta, float *dA_log, void *dB, void *dC,
                   float *dD, void *dz, float *ddelta_bias, float *dinitial_state,
                   int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Training pair: a forward that keeps what the backward needs, and a
 * backward that starts from it instead of running the forward scan again.
 *
 * ss_scan_checkpoint_bytes: bytes of the checkpoint buffer for these sizes,
 * b * ((L - 1) / 8) * n * d_in * 4 (0 for invalid sizes, and 0 for L <= 8).
 *
 * ss_scan_fwd_save: ss_scan_fwd_ex (same arguments, results and workspace)
 * that also writes
 *   checkpoints : (b, (L - 1) / 8, n, d_in) fp32, the state after steps
 *                 8, 16, ... (checkpoint i holds h after step 8 (i + 1));
 *                 required (SS_ERR_NULL), 4-byte aligned
 *   y_pre       : (b, L, d_in) dtype, the readout sum_k C h + D u before the
 *                 gate; required when z is given (SS_ERR_NULL), else ignored
 * n <= SS_MAX_BWD_STATE.  Neither may overlap an input, another output or
 * the workspace (SS_ERR_ALIAS).
 *
 * ss_scan_bwd_saved: ss_scan_bwd_ex (same arguments and results) given the
 * checkpoints and y_pre of an ss_scan_fwd_save call on the same inputs; it
 * does not run the forward scan again and forms dz from y_pre.  Its
 * workspace is ss_scan_bwd_saved_workspace_bytes() long (smaller than
 * ss_scan_bwd's: no room for a forward pass or checkpoints) and 256-byte
 * aligned.  Results agree with ss_scan_bwd_ex: bit for bit with fp32
 * inputs; with bf16 inputs dz takes y_pre rounded to bf16 where ss_scan_bwd
 * uses it unrounded.  The checkpoints (for L > 8) and y_pre are not written.
 * Returns an ss_status.
 */
size_t ss_scan_checkpoint_bytes(int64_t b, int64_t L, int64_t d_in, int64_t n);

size_t ss_scan_bwd_saved_workspace_bytes(int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype);

int ss_scan_fwd_save(const void *u, const void *delta, const float *A_log,
                     const void *B, const void *C, const float *D,
                     const void *z, const float *delta_bias, int delta_softplus,
                     const float *initial_state, int discretization,
                     void *y, float *last_state, float *checkpoints, void *y_pre,
                     int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype,
                     void *workspace, size_t workspace_bytes, void *stream);

int ss_scan_bwd_saved(const void *u, const void *delta, const float *A_log,
                      const void *B, const void *C, const float *D,
                      const void *z, const float *delta_bias, int delta_softplus,
                      const float *initial_state, int discretization,
                      const float *checkpoints, const void *y_pre,
                      const void *dy, const float *dlast_state,
                      void *du, void *ddelta, float *dA_log, void *dB, void *dC,
                      float *dD, void *dz, float *ddelta_bias, float *dinitial_state,
                      int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Largest convolution width W of ss_conv_update. */
#define SS_MAX_CONV_WIDTH 8

/*
 * The convolution step that precedes the SSM step of a decode step
 * (jiafeimiao.top page, Mamba.step, "Conv step": the causal depthwise
 * convolution of the block applied to one new token).  Per (b, d) channel:
 *     window[0 .. W-2] = window[1 .. W-1];  window[W-1] = x[b, d]
 *     out[b, d] = sum_w window[w] * weight[d, w] + bias[d]      (bias optional)
 *     out[b, d] = silu(out[b, d])                               (when silu != 0)
 *
 *   conv_state : (b, d_in, W)  dtype, the window, read and overwritten in place
 *   x          : (b, d_in)     dtype, the new input
 *   weight     : (d_in, W)     fp32 (the conv1d weight (d_in, 1, W) without its middle axis)
 *   bias       : (d_in)        fp32, or NULL
 *   silu       : nonzero -> apply silu to the output
 *   out        : (b, d_in)     dtype, output (the x of the SSM step, after
 *                              the caller's projections have produced dt, B, C from it)
 * Sizes: b, d_in >= 1, b * d_in < 2^28, 1 <= W <= SS_MAX_CONV_WIDTH
 * (else SS_ERR_SHAPE / SS_ERR_UNSUPPORTED).  out must not overlap any input
 * and conv_state must not overlap x, weight or bias (SS_ERR_ALIAS).
 * Returns an ss_status.
 */
int ss_conv_update(void *conv_state, const void *x, const float *weight,
                   const float *bias, int silu, void *out,
                   int64_t b, int64_t d_in, int64_t W, int dtype, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *ss_status_string(int status);

/*
 * For tests and tuning only; never needed for correct results.  Overrides,
 * process-wide and for every later call, how the scans split their work
 * (each argument 0 = the library's own choice):
 *   segments      : cut L into this many segments (1..16)
 *   waves         : 4 = 4 recurrence waves of 4 states at 9 <= n <= 16
 *   time_parallel : 1 = the time-parallel forward kernel for n <= 2
 *                   (Euler input term, zero initial state)
 *   spin_limit    : polls before a segment wait gives up
 *   wait_never    : 1 = segment waits poll a word nothing sets, so each
 *                   gives up after spin_limit polls (exercises SS_ERR_TIMEOUT)
 * Results agree with the default within the stated tolerances (the order of
 * fp32 additions may change) and are deterministic for each setting.
 * Returns SS_OK, or SS_ERR_SHAPE for an argument out of range.
 */
int ss_set_test_plan(int segments, int waves, int time_parallel, int spin_limit, int wait_never);

#ifdef __cplusplus
}
#endif

#endif /* SS_SCAN_H */
