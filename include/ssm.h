/*
 * ssm.h -- C ABI of the MI355X (gfx950) selective state-space scan library.
 *
 * Two operations, both run by hand-written HIP kernels on the caller's stream:
 *
 *   ssm_scan_fwd      the selective scan (S6) forward over a whole sequence;
 *   ssm_state_update  one single-token decode step of the same recurrence.
 *
 * What is computed (per batch b and channel d, independently; N = dstate):
 *
 *   dt_t  = softplus(delta[b,t,d] + delta_bias[d])   if delta_softplus
 *         = delta[b,t,d] + delta_bias[d]              otherwise
 *   h_t   = exp(dt_t * A[d,:]) (.) h_{t-1} + dt_t * B[b,t,:] * x[b,t,d],   h_{-1} = 0
 *   y_t   = <C[b,t,:], h_t> + D[d] * x[b,t,d]
 *   y_t  *= silu(z[b,t,d])                            if z is given
 *
 * Sources (page title and section):
 *  - "Mamba 论文精读" (youngju.dev), sec. 2.2: the discretised recurrence
 *    h_t = Abar h_{t-1} + Bbar x_t, y_t = C h_t with Abar = exp(delta A);
 *    sec. 3.3: selective_scan(x, delta, A, B, C) with x, delta (B,L,D),
 *    A (D,N), B and C (B,L,N) shared across channels, Bbar x = delta B x,
 *    a zero initial state, and the state updated before y_t is read out;
 *    sec. 3.1: delta = softplus(Linear_delta(x)), whose projection carries a
 *    bias (sec. 3.4); sec. 3.4: the per-channel skip D and the SiLU(z) gate;
 *    sec. 6: decoding costs O(1) per token with a fixed-size state.
 *  - "Mamba的基础知识" (weblog-19d), state space model section: D is the
 *    direct input-to-output term.
 *  - "mamba->jamba" (blog.csdn.net), sec. 2.3: discretisation, scan and
 *    read-out are fused on chip and the (B,L,D,N) intermediates never reach
 *    HBM; only the final state is written.
 *
 * Conventions shared by every call
 *  - Every tensor argument is a DEVICE pointer to contiguous row-major memory
 *    in the shape listed beside it (last dimension fastest).  The caller owns
 *    every buffer; the library keeps no pointer after a call returns.
 *  - `dtype` is the storage type of x, delta, B, C, z and y.  A, D,
 *    delta_bias, last_state and state are always fp32.  All arithmetic is
 *    fp32; bf16 results are rounded to nearest-even.
 *  - Optional arguments are NULL: D (no skip term), z (no gate), delta_bias
 *    (zero bias), last_state (not written).
 *  - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t;
 *    NULL = the null stream) and the call returns.  A non-OK status means
 *    nothing was enqueued, except SSM_ERR_HIP, which reports a failed launch
 *    (work enqueued before it may still run).  Faults inside a kernel
 *    surface at the caller's next synchronisation.
 *  - Validation happens on the host before any launch: negative sizes,
 *    NULL required pointers and overlapping outputs give
 *    SSM_ERR_INVALID_ARG; a dstate outside {1, 2, 4, 8, 16, 32, 64} or an
 *    unknown dtype gives SSM_ERR_UNSUPPORTED; a pointer not aligned to its
 *    element size gives SSM_ERR_MISALIGNED (and for ssm_scan_fwd with bf16
 *    and an even dstate, B and C must be 4-byte aligned, since they are read
 *    as bf16 pairs).  Faster paths are used when x, delta, z and y are
 *    16-byte aligned and dim is a multiple of 8 (bf16) or 4 (fp32); other
 *    layouts are handled element by element.  A batch, seqlen or dim of 0 is
 *    valid and enqueues nothing (except that ssm_scan_fwd zero-fills a
 *    non-empty last_state when seqlen == 0, the state after no steps).
 *  - No C++ exception crosses the ABI.  The calls are thread-safe; calls
 *    that write the same buffers must be ordered by the caller.
 *  - ssm_last_error() gives a thread-local human-readable detail for the
 *    last non-OK status returned on the calling thread.
 */
#ifndef SSM_H_
#define SSM_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 2

#if defined(__GNUC__)
#define SSM_API __attribute__((visibility("default")))
#else
#define SSM_API
#endif

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype_t;

typedef enum {
  SSM_OK = 0,
  SSM_ERR_INVALID_ARG = 1,
  SSM_ERR_UNSUPPORTED = 2,
  SSM_ERR_MISALIGNED = 3,
  SSM_ERR_HIP = 4
} ssm_status_t;

/*
 * Selective scan forward over a whole sequence ("Mamba 论文精读" sec. 3.3;
 * "mamba->jamba" sec. 2.3 for the fused, on-chip evaluation).
 *
 *   x, delta, z   (batch, seqlen, dim)    dtype; delta is the raw step
 *   A             (dim, dstate)           fp32, expected negative (not checked)
 *   B, C          (batch, seqlen, dstate) dtype, shared by all channels
 *   D, delta_bias (dim)                   fp32, or NULL
 *   y             (batch, seqlen, dim)    dtype, written; must not overlap an input
 *   last_state    (batch, dim, dstate)    fp32 h after the last step, or NULL
 *
 * For small batch*dim the sequence is split into segments scanned in
 * parallel and joined by a carry pass; that needs (segments * batch * dim *
 * (dstate + 1)) fp32 of device scratch.  The library keeps one such buffer
 * per (device, stream), allocated with hipMalloc on first need and replaced
 * by a larger one when a larger call needs it.  A replaced buffer is never
 * freed (work already enqueued, or a graph captured earlier, may still hold
 * its address); it stays allocated until the process ends.  A call that
 * would allocate must not be captured into a HIP graph; calls on one stream
 * reuse its buffer in stream order, and calls on different streams never
 * share one.
 */
SSM_API ssm_status_t ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                          const void *x, const void *delta, const float *A, const void *B, const void *C,
                          const float *D, const void *z, const float *delta_bias, int delta_softplus, void *y,
                          float *last_state, void *stream);

/*
 * The discretised input term Bbar x.
 *   SSM_BBAR_DELTA_B  Bbar = Delta B (the default; the simplified
 *                     selective_scan of "Mamba 论文精读" sec. 3.3)
 *   SSM_BBAR_ZOH      the exact zero-order hold of sec. 2.2,
 *                     Bbar = (Delta A)^-1 (exp(Delta A) - I) Delta B, i.e.
 *                     (exp(Delta A_n) - 1) / A_n B_n for the diagonal A
 *                     (Delta B_n where A_n = 0).  About 2.5x the arithmetic
 *                     of the default; the backward pass supports only the
 *                     default.
 */
typedef enum { SSM_BBAR_DELTA_B = 0, SSM_BBAR_ZOH = 1 } ssm_bbar_mode_t;

/*
 * How the scan's work is laid out over a workgroup (the result is the same
 * bits either way: both compute each step in the same order).
 *   SSM_LAYOUT_AUTO           the library chooses;
 *   SSM_LAYOUT_CHANNEL_LANES  lane = channel, each scan wave one range of
 *                             state indices of 64 channels, the per-(t, d)
 *                             work on waves next to every scan wave; every
 *                             dstate, both Bbar modes, the sequence split;
 *   SSM_LAYOUT_STATE_ROWS     a scan wave holds 16 channels x 16 state
 *                             indices (one 16-lane row per 4 states), the
 *                             per-(t, d) work on a SIMD of its own, and
 *                             16 x channel_groups channels per workgroup:
 *                             dstate 16, SSM_BBAR_DELTA_B and one segment
 *                             only (else SSM_ERR_UNSUPPORTED);
 *   SSM_LAYOUT_TIME_SCAN      time parallel inside a chunk: one workgroup per
 *                             (batch row, channel), each lane a block of 4 or
 *                             8 steps (chunk_steps 256 or 512), the blocks
 *                             joined by a wave64 associative scan of
 *                             (abar, state) pairs ("mamba->jamba" sec. 2.3)
 *                             and a carry across chunks; for few channels and
 *                             long sequences.  Never chosen automatically:
 *                             measured slower than the sequence split.  Same
 *                             limits as SSM_LAYOUT_STATE_ROWS.
 */
typedef enum {
  SSM_LAYOUT_AUTO = 0,
  SSM_LAYOUT_CHANNEL_LANES = 1,
  SSM_LAYOUT_STATE_ROWS = 2,
  SSM_LAYOUT_TIME_SCAN = 3
} ssm_scan_layout_t;

/*
 * Launch-shape overrides for ssm_scan_fwd.  Every field 0 means "choose
 * automatically".  The result does not depend on these choices beyond fp32
 * rounding of the re-associated cross-segment carry; they exist for tuning
 * and for the invariance tests.
 *   chains_per_lane  state chains (values of n) per GPU lane: 1, 2, 4, 8 or 16,
 *                    dividing dstate;
 *   segments         number of sequence segments scanned in parallel (>= 1);
 *   chunk_steps      time steps staged per LDS tile: 16 or 32 (32 needs at most
 *                    4 scan waves, i.e. dstate / chains_per_lane <= 4, and
 *                    bbar_mode SSM_BBAR_DELTA_B; with SSM_LAYOUT_STATE_ROWS it
 *                    needs channel_groups <= 3).
 *   bbar_mode        the discretised input term (not a launch-shape choice:
 *                    it changes the result), see ssm_bbar_mode_t.
 *   layout           ssm_scan_layout_t;
 *   channel_groups   with SSM_LAYOUT_STATE_ROWS: scan waves (groups of 16
 *                    channels) per workgroup, 1 to 6.
 * chains_per_lane applies to SSM_LAYOUT_CHANNEL_LANES only (the state rows
 * always hold 4 chains per lane).  reserved must be zero.
 */
typedef struct {
  int32_t chains_per_lane;
  int32_t segments;
  int32_t chunk_steps;
  int32_t bbar_mode;
  int32_t layout;
  int32_t channel_groups;
  int32_t reserved[2];
} ssm_scan_opts_t;

/* ssm_scan_fwd with launch-shape overrides (opts may be NULL). An override
 * the kernels cannot honour gives SSM_ERR_UNSUPPORTED. */
SSM_API ssm_status_t ssm_scan_fwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                             const void *x, const void *delta, const float *A, const void *B, const void *C,
                             const float *D, const void *z, const float *delta_bias, int delta_softplus,
                             void *y, float *last_state, void *stream, const ssm_scan_opts_t *opts);

/*
 * ssm_scan_fwd_ex for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, layouts, validation and results as ssm_scan_fwd_ex (the
 * same kernels run, so the outputs are bit-identical); it calls no hipMalloc,
 * hipFree or other allocating routine.
 *
 * The split-sequence path's segment summaries (segments * batch * dim *
 * (dstate + 1) fp32, see ssm_scan_fwd) go to a file-scope device array of
 * 2^22 fp32 (16 MiB) that each GPU the library runs on holds until the
 * process ends.  A call that needs more gives SSM_ERR_UNSUPPORTED before any
 * launch; the automatic launch shape needs at most about 2.8 M fp32 for every
 * supported dstate, so only forced segment counts (opts->segments) on large
 * batch * dim can exceed it.  Nothing in the array needs to start at zero:
 * every call writes each summary before reading it.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that may overlap on one GPU (different streams, or
 * different host threads, without ordering between them) race on it and
 * give wrong results.  Order them on one stream, or use ssm_scan_fwd_ex.
 * The first call on a device looks the array's address up
 * (hipGetSymbolAddress) and caches it; an error there gives SSM_ERR_HIP.
 */
SSM_API ssm_status_t ssm_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                  ssm_dtype_t dtype, const void *x, const void *delta, const float *A,
                                  const void *B, const void *C, const float *D, const void *z,
                                  const float *delta_bias, int delta_softplus, void *y, float *last_state,
                                  void *stream, const ssm_scan_opts_t *opts);

/*
 * One single-token decode step ("Mamba 论文精读" sec. 6: O(1) work per token
 * with a fixed-size state; sec. 2.2: the recurrence).
 *
 *   state         (batch, dim, dstate)    fp32, read and updated in place
 *   x, delta, z   (batch, dim)            dtype
 *   A             (dim, dstate)           fp32
 *   B, C          (batch, dstate)         dtype
 *   D, delta_bias (dim)                   fp32, or NULL
 *   y             (batch, dim)            dtype, written; must not overlap state or an input
 *
 * Running it for t = 0..L-1 from a zero state gives the same y_t and final
 * state as ssm_scan_fwd over those L steps.
 */
SSM_API ssm_status_t ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, ssm_dtype_t dtype, float *state,
                              const void *x, const void *delta, const float *A, const void *B, const void *C,
                              const float *D, const void *z, const float *delta_bias, int delta_softplus, void *y,
                              void *stream);

/*
 * Backward pass of ssm_scan_fwd (zero initial state): the gradients of
 * sum(dy * y) with respect to every input.  The forward states are
 * recomputed, never stored per step ("mamba->jamba" sec. 2.3: the backward
 * recomputes Abar and Bbar, as FlashAttention recomputes its scores).
 *
 *   inputs: as ssm_scan_fwd, plus dy (batch, seqlen, dim) dtype
 *   dx, ddelta, dz (batch, seqlen, dim) dtype;  dB, dC (batch, seqlen, dstate) dtype
 *   dA (dim, dstate), dD (dim), ddelta_bias (dim) fp32
 *   dz is required when z is given (else ignored), dD when D is given,
 *   ddelta_bias when delta_bias is given; ddelta is the gradient with respect
 *   to the raw delta (before bias and softplus).
 *
 * dstate must be 1, 2, 4, 8, 16, 32 or 64.  last_state is not
 * differentiated.  The batch sums of dA / dD / ddelta_bias are taken in a
 * fixed order.  With the channel-lane layout the channel sums of dB / dC are
 * too, so the result does not vary from run to run; the state-row layout
 * (ssm_bwd_opts_t, chosen automatically for bf16 dstate 16) adds them with
 * atomics.  Scratch, in the same per-(device, stream) buffer as the
 * split-sequence scan (same rules as ssm_scan_fwd), in fp32 values:
 *   channel lanes, with T = 16 (dstate <= 16), 8 (dstate 32) or 4 (dstate
 *   64), halved for SSM_BBAR_ZOH but at least 4: batch*ceil(seqlen/T)*dstate*dim
 *   + 2*ceil(dim/64)*batch*seqlen*dstate + batch*dstate*dim + 2*T*batch*dim;
 *   state rows, with T = 32: batch*ceil(seqlen/T)*16*dim + 2*batch*seqlen*16
 *   + batch*16*dim + 2*T*batch*dim.
 */
SSM_API ssm_status_t ssm_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                                  const void *x, const void *delta, const float *A, const void *B, const void *C,
                                  const float *D, const void *z, const float *delta_bias, int delta_softplus,
                                  const void *dy, void *dx, void *ddelta, float *dA, void *dB, void *dC, float *dD,
                                  void *dz, float *ddelta_bias, void *stream);

/* Options of ssm_scan_bwd_ex: bbar_mode as in ssm_scan_opts_t (the forward
 * being differentiated); layout (ssm_scan_layout_t) picks the work
 * decomposition:
 *   SSM_LAYOUT_AUTO           state rows where they apply, else channel lanes;
 *   SSM_LAYOUT_CHANNEL_LANES  one channel per lane, 64 channels per workgroup,
 *                             every dtype / dstate / bbar_mode;
 *   SSM_LAYOUT_STATE_ROWS     16 channels x 16 states per wave, 48 channels
 *                             per workgroup, 32-step chunks: bf16 only,
 *                             dstate 16, SSM_BBAR_DELTA_B, dim a multiple of 8
 *                             and x, delta, z, dy, dx, ddelta, dz, B, C
 *                             16-byte aligned (else SSM_ERR_UNSUPPORTED).
 *                             Its dB / dC channel sums are added with
 *                             atomics, so their last bits may vary from run
 *                             to run; every other gradient is summed in a
 *                             fixed order.
 * SSM_LAYOUT_TIME_SCAN is a forward-only layout (SSM_ERR_UNSUPPORTED).
 * reserved must be zero. */
typedef struct {
  int32_t bbar_mode;
  int32_t layout;
  int32_t reserved[6];
} ssm_bwd_opts_t;

/*
 * ssm_scan_bwd for either input term (opts may be NULL: SSM_BBAR_DELTA_B).
 * With SSM_BBAR_ZOH it differentiates the exact zero-order-hold forward of
 * "Mamba 论文精读" sec. 2.2: with phi = expm1(Delta A) / A the input term is
 * phi B x, dphi/dDelta = exp(Delta A) and dphi/dA = (Delta exp(Delta A) -
 * phi) / A.  Same arguments, layouts, scratch and errors as ssm_scan_bwd.
 */
SSM_API ssm_status_t ssm_scan_bwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                             const void *x, const void *delta, const float *A, const void *B, const void *C,
                             const float *D, const void *z, const float *delta_bias, int delta_softplus,
                             const void *dy, void *dx, void *ddelta, float *dA, void *dB, void *dC, float *dD,
                             void *dz, float *ddelta_bias, void *stream, const ssm_bwd_opts_t *opts);

/*
 * A training pair that hands the forward's states to the backward.  The
 * backward recomputes the states of each 32-step chunk from the state that
 * enters it ("mamba->jamba" sec. 2.3: recompute instead of storing every
 * step); with these two calls the forward stores those entering states, so
 * the backward does not run the forward recurrence again (and reads x and
 * delta once instead of twice).
 *
 *   checkpoints  (batch, ceil(seqlen / 32), dim, dstate) fp32: entry [b][c]
 *                is the state before step 32 c in last_state's layout (entry
 *                0 is zero).  Written by ssm_scan_fwd_ckpt, read by
 *                ssm_scan_bwd_ckpt; owned by the caller; must not overlap any
 *                other argument (else SSM_ERR_INVALID_ARG), 16-byte aligned
 *                (else SSM_ERR_MISALIGNED), and not NULL when there is work.
 *
 * ssm_scan_fwd_ckpt: ssm_scan_fwd plus the checkpoints.  It runs the
 * state-row layout, so dstate must be 16 (else SSM_ERR_UNSUPPORTED); y and
 * last_state are bit-identical to ssm_scan_fwd_ex with SSM_LAYOUT_STATE_ROWS.
 * ssm_scan_bwd_ckpt: ssm_scan_bwd (SSM_BBAR_DELTA_B) from the checkpoints of
 * ssm_scan_fwd_ckpt on the same inputs.  It runs the state-row backward, so
 * it needs bf16, dstate 16, dim a multiple of 8 and 16-byte aligned x, delta,
 * z, dy, dx, ddelta, dz, B, C (else SSM_ERR_UNSUPPORTED).  Scratch as the
 * state-row backward of ssm_scan_bwd without its first term.  Nothing checks
 * that the checkpoints come from the same inputs: others give the gradients
 * of a different forward.
 */
SSM_API ssm_status_t ssm_scan_fwd_ckpt(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                                       const void *x, const void *delta, const float *A, const void *B,
                                       const void *C, const float *D, const void *z, const float *delta_bias,
                                       int delta_softplus, void *y, float *last_state, float *checkpoints,
                                       void *stream);
SSM_API ssm_status_t ssm_scan_bwd_ckpt(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                                       const void *x, const void *delta, const float *A, const void *B,
                                       const void *C, const float *D, const void *z, const float *delta_bias,
                                       int delta_softplus, const void *dy, void *dx, void *ddelta, float *dA,
                                       void *dB, void *dC, float *dD, void *dz, float *ddelta_bias,
                                       const float *checkpoints, void *stream);

/*
 * Depthwise causal convolution that feeds the scan in the Mamba block
 * ("Mamba 论文精读" sec. 3.4, MambaBlock: Conv1d with one group per channel,
 * kernel width K and K-1 zeros of padding, the first L outputs kept, then
 * SiLU).  For each batch row b and channel d:
 *
 *   y[b,t,d] = bias[d] + sum_{k<K} weight[d,k] * xin[t-(K-1)+k]
 *   xin[s]   = x[b,s,d] for s >= 0, initial_state[b,d,(K-1)+s] for s < 0
 *              (zeros when initial_state is NULL)
 *   y        = silu(y) when silu != 0
 *   final_state[b,d,j] = xin[L-(K-1)+j], j = 0..K-2 (the last K-1 inputs,
 *              oldest first): pass it as the next call's initial_state, or
 *              as the conv_state of ssm_causal_conv1d_update.
 *
 *   x, y          (batch, seqlen, dim)  dtype (the scan's x layout)
 *   weight        (dim, width)          fp32, width in 1..4
 *   bias          (dim)                 fp32, or NULL
 *   initial_state (batch, dim, width-1) dtype, or NULL
 *   final_state   (batch, dim, width-1) dtype, or NULL; written
 *
 * Outputs must not overlap an input or each other.  The kernel is
 * bandwidth-bound: x is read once and y written once.
 */
SSM_API ssm_status_t ssm_causal_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                                           ssm_dtype_t dtype, const void *x, const float *weight, const float *bias,
                                           const void *initial_state, int silu, void *y, void *final_state,
                                           void *stream);

/*
 * One token of the same convolution: the window is conv_state[b,d,0..K-2]
 * followed by x[b,d]; y = bias + sum weight * window (then SiLU when asked);
 * conv_state then drops its oldest input and appends x (in place).
 *
 *   conv_state (batch, dim, width-1) dtype, read and updated (may be NULL when width == 1)
 *   x, y       (batch, dim)          dtype
 *   weight     (dim, width) fp32; bias (dim) fp32 or NULL
 *
 * Running it over x[:, t] for t = 0..L-1 gives ssm_causal_conv1d_fwd's
 * outputs and final state for the same initial state.
 */
SSM_API ssm_status_t ssm_causal_conv1d_update(int64_t batch, int64_t dim, int64_t width, ssm_dtype_t dtype,
                                              void *conv_state, const void *x, const float *weight,
                                              const float *bias, int silu, void *y, void *stream);

/* Options of ssm_state_update_ex: bbar_mode as in ssm_scan_opts_t; reserved
 * must be zero. */
typedef struct {
  int32_t bbar_mode;
  int32_t reserved[7];
} ssm_update_opts_t;

/* ssm_state_update with options (opts may be NULL: the defaults). */
SSM_API ssm_status_t ssm_state_update_ex(int64_t batch, int64_t dim, int64_t dstate, ssm_dtype_t dtype, float *state,
                                         const void *x, const void *delta, const float *A, const void *B,
                                         const void *C, const float *D, const void *z, const float *delta_bias,
                                         int delta_softplus, void *y, void *stream, const ssm_update_opts_t *opts);

/* Options of ssm_ssd_fwd.  head_slice: head channels per workgroup (16, 32
 * or 64, dividing headdim), or 0 for the largest one the library has for
 * this dstate and headdim.  segments: pieces the sequence is cut into (each
 * a whole number of 64-step chunks; 1 = none, 0 = chosen by the library:
 * enough to give every compute unit a workgroup when the batch rows and
 * heads alone cannot).  gram: where each chunk's C B^T (the Gram matrix the
 * heads of a group share, "Mamba 论文精读" sec. 4.2) is computed: 1 = once
 * per (batch row, group, chunk) by a separate pass whose tiles every head's
 * workgroup then reads (64-channel slices only, else SSM_ERR_UNSUPPORTED),
 * -1 = inside every head's workgroup, 0 = chosen by the library (the
 * separate pass when at least 4 workgroups share a group's B and C and each
 * runs at least 8 chunks).  The outputs are the same bits either way.
 * reserved must be zero. */
typedef struct {
  int32_t head_slice;
  int32_t segments;
  int32_t gram;
  int32_t reserved[5];
} ssm_ssd_opts_t;

/*
 * Mamba-2 state space dual (SSD) layer, forward ("Mamba 论文精读" sec. 4.1:
 * the recurrence h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t and its dual, a
 * product with a causal semi-separable matrix; sec. 4.2: multiple heads and
 * larger states; sec. 5.2: the Mamba2 layer with headdim and d_state).  A is
 * one scalar per head, Bbar = dt B as in ssm_scan_fwd, and the heads of a
 * group (nheads / ngroups consecutive heads) share B and C.  For batch row
 * b, head h in group g and head channel p, from S = initial_state[b,h,p,:]
 * (zero when NULL):
 *
 *   dt_t = softplus(dt[b,t,h] + dt_bias[h])   (no softplus when dt_softplus == 0)
 *   S    = exp(dt_t A[h]) S + dt_t x[b,t,h,p] B[b,t,g,:]
 *   y[b,t,h,p] = (C[b,t,g,:] . S + D[h] x[b,t,h,p]) * silu(z[b,t,h,p])
 *   final_state[b,h,p,:] = S after the last step
 *
 *   x, z, y        (batch, seqlen, nheads, headdim)  bf16; z may be NULL
 *   dt             (batch, seqlen, nheads)           bf16
 *   B, C           (batch, seqlen, ngroups, dstate)  bf16
 *   A              (nheads) fp32;  D, dt_bias (nheads) fp32 or NULL
 *   initial_state  (batch, nheads, headdim, dstate)  fp32 state entering the
 *                  sequence, or NULL (zero): the final state of an earlier call
 *                  continues it
 *   final_state    (batch, nheads, headdim, dstate)  fp32, or NULL
 *
 * The sequence is taken in chunks of 64 steps whose products run on bf16
 * matrix cores with fp32 accumulation; the state carried between chunks is
 * fp32 and is rounded to bf16 only as an operand of the chunk's read-out.
 * With a sequence split the segments' states go to the same per-(device,
 * stream) scratch as the split-sequence scan: (segments-1)*batch*nheads*
 * headdim*dstate + segments*batch*nheads fp32 (same rules as ssm_scan_fwd);
 * the separate C B^T pass adds batch*ngroups*ceil(seqlen/64)*3072 fp32 to it
 * (12 KB per chunk).
 * Storage must be bf16 (SSM_F32 gives SSM_ERR_UNSUPPORTED).  dstate must be
 * 32, 64, 128 or 256 and headdim a multiple of 16; workgroups take 16-, 32-
 * or 64-channel slices of a head, dstate 128 only 32 or 64 and dstate 256
 * only 64, so dstate 256 needs headdim a multiple of 64 and dstate 128 one of
 * 32 (else SSM_ERR_UNSUPPORTED).
 * x, z, y, B, C, initial_state and final_state must be 16-byte aligned
 * (else SSM_ERR_MISALIGNED).  Outputs must not overlap an input or each
 * other.  opts may be NULL.
 */
SSM_API ssm_status_t ssm_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                                 int64_t ngroups, ssm_dtype_t dtype, const void *x, const void *dt, const float *A,
                                 const void *B, const void *C, const float *D, const void *z,
                                 const float *dt_bias, int dt_softplus, const float *initial_state, void *y,
                                 float *final_state, void *stream, const ssm_ssd_opts_t *opts);

/*
 * One token of the same layer, the recurrent view of "Mamba 论文精读" sec.
 * 4.1 (O(1) work per token): for batch row b, head h in group g, channel p,
 *
 *   dt = softplus(dt[b,h] + dt_bias[h])   (no softplus when dt_softplus == 0)
 *   state[b,h,p,:] = exp(dt A[h]) state[b,h,p,:] + dt x[b,h,p] B[b,g,:]
 *   y[b,h,p] = (C[b,g,:] . state[b,h,p,:] + D[h] x[b,h,p]) * silu(z[b,h,p])
 *
 *   state      (batch, nheads, headdim, dstate) fp32, updated in place
 *              (16-byte aligned)
 *   x, z, y    (batch, nheads, headdim) bf16; z may be NULL
 *   dt         (batch, nheads) bf16
 *   B, C       (batch, ngroups, dstate) bf16 (8-byte aligned)
 *   A, D, dt_bias (nheads) fp32; D and dt_bias may be NULL
 *
 * Running it over the tokens of a sequence from an initial state gives
 * ssm_ssd_fwd's outputs and final state for that initial state (up to the
 * rounding of the chunked products).  dstate must be 32, 64, 128 or 256;
 * storage bf16.
 */
SSM_API ssm_status_t ssm_ssd_state_update(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                                          int64_t ngroups, ssm_dtype_t dtype, float *state, const void *x,
                                          const void *dt, const float *A, const void *B, const void *C,
                                          const float *D, const void *z, const float *dt_bias, int dt_softplus,
                                          void *y, void *stream);

/* Static string naming a status code ("SSM_OK", ...); never NULL. */
SSM_API const char *ssm_status_string(ssm_status_t status);

/* Thread-local detail for the last non-OK status on this thread ("" if none).
 * Valid until the next library call on the same thread. */
SSM_API const char *ssm_last_error(void);

/* SSM_ABI_VERSION of the loaded library. */
SSM_API int ssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H_ */
