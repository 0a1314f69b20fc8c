/*
 * ssm.h -- C ABI of libssm.so, the gfx950 (MI355X) selective-scan library.
 *
 * Four operations, all from the Mamba pages (cited by page title and section):
 *
 *   ssm_selective_scan_fwd  -- prefill.  For every batch row b, channel d and
 *     state index n, with Delta_t = softplus(delta_t + bias[d]) (Mamba paper
 *     notes, 0539edu.com, section 2.3; Mamba training/inference guide, FAQ 2):
 *         h_t[n] = exp(Delta_t * A[d,n]) * h_{t-1}[n] + Delta_t * B[b,g,n,t] * u_t
 *         y_t    = sum_n C[b,g,n,t] * h_t[n] + D[d] * u_t
 *         out_t  = y_t * silu(z_t)
 *     where g is the B/C group of channel d (one group: B_t and C_t shared
 *     by every channel, the layout of the pages).
 *     starting from h_{-1} = h0 (or 0), and optionally returning h_{L-1}.
 *     The discrete recurrence and readout are section 2.2 of the Mamba model
 *     notes; the per-channel diagonal SSM is section 4.4 there; B, C and
 *     Delta depending on the token is section 4.1; the gate is the block's
 *     gate branch (section 4.3).
 *
 *   ssm_selective_scan_bwd -- the gradients of the prefill scan, i.e. its
 *     reverse-mode derivative.  Back-propagation needs the state at every
 *     step; as the Mamba paper notes advise (section 5.4: gradient
 *     checkpointing, state passed at chunk edges), the forward keeps only one
 *     state per 16-token chunk and the backward recomputes the steps between.
 *
 *   ssm_ssd_scan_fwd -- the Mamba-2 SSM (multi-head, scalar decay per head,
 *     the SSD layer) prefill; see ssm_ssd_args.
 *   ssm_selective_state_update -- decode: the same recurrence for a single
 *     token, reading and writing a resident fp32 state (Mamba paper notes,
 *     section 4.3: inference keeps one fixed-size state and updates it once
 *     per generated token).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates and never frees; its only global state is the
 *     static scratch of ssm_selective_scan_fwd_noalloc (and the per-device
 *     address of it), which no other entry point touches.
 *   - Strides are in ELEMENTS and must be >= 0.  The innermost (time, or
 *     state for decode) stride is implicitly 1.
 *   - io_dtype (SSM_F32 or SSM_BF16) is the dtype of u/delta/z/B/C/out in the
 *     scan and of x/dt/z/B/C/out in decode.  A, D, the Delta bias, h0,
 *     last_state and the decode state are always fp32.
 *   - All arithmetic is fp32; bf16 inputs are widened exactly; fp32 results
 *     are rounded to bf16 to nearest-even when io_dtype is SSM_BF16.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream).  The return value covers host-side validation and the launch
 *     itself; a device fault shows up at the caller's next synchronisation.
 *   - No exception crosses the ABI; errors are ssm_status codes, explained by
 *     ssm_status_string().  On any error nothing is launched.
 *   - The library is re-entrant and thread-safe (the no-allocation scan's
 *     shared scratch excepted, see there).
 */
#ifndef SSM_H_
#define SSM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 8

/* Tokens between two state checkpoints (see ssm_scan_args.checkpoints). */
#define SSM_CHECKPOINT_TOKENS 16

/* Largest width of the fused causal conv (see ssm_scan_args.conv_weight). */
#define SSM_MAX_CONV 8

/* Largest state size of the scan and the decode update (the Mamba paper
 * notes, section 3.2, put d_state between 8 and 64). */
#define SSM_MAX_DSTATE 64

/* Size of the static device scratch of ssm_selective_scan_fwd_noalloc. */
#define SSM_NOALLOC_SCRATCH_BYTES (32u << 20)

typedef enum ssm_status {
  SSM_OK = 0,
  SSM_ERR_NULL = 1,        /* a required pointer is NULL                       */
  SSM_ERR_SHAPE = 2,       /* negative size, dstate < 1, or ngroups not
                              dividing dim                                     */
  SSM_ERR_STRIDE = 3,      /* negative stride                                  */
  SSM_ERR_DTYPE = 4,       /* io_dtype is not SSM_F32 / SSM_BF16               */
  SSM_ERR_ALIGN = 5,       /* pointer not aligned to its element size          */
  SSM_ERR_ALIAS = 6,       /* an output overlaps an input it must not overlap  */
  SSM_ERR_UNSUPPORTED = 7, /* valid but not built: dstate > SSM_MAX_DSTATE
                              (backward: also groups that split a block of
                              16 channels), seqlen too large for
                              32-bit token indices (>= 2^31 - 64), or row
                              spans past the 32-bit windows (see
                              ssm_scan_args)                                   */
  SSM_ERR_HIP = 8,         /* the HIP runtime rejected the launch              */
  SSM_ERR_SCRATCH = 9      /* ssm_selective_scan_fwd_noalloc: the segment
                              scratch exceeds SSM_NOALLOC_SCRATCH_BYTES        */
} ssm_status;

typedef enum ssm_dtype { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/* Arguments of the prefill scan.
 *   u, delta, z, out : (batch, dim, seqlen), time stride 1; element (b, d, t)
 *                      at ptr[b * *_batch_stride + d * *_dim_stride + t].
 *   B, C             : (batch, ngroups, dstate, seqlen), time stride 1;
 *                      element (b, g, n, t) at ptr[b * *_batch_stride +
 *                      g * *_group_stride + n * *_state_stride + t].  Channel
 *                      d reads group d / (dim / ngroups); ngroups 0 or 1 is
 *                      one group shared by all channels (group stride
 *                      unused), ngroups == dim gives every channel its own.
 *   A                : (dim, dstate) fp32, element (d, n) at
 *                      A[d * A_dim_stride + n * A_state_stride].
 *   D, delta_bias    : (dim) fp32, contiguous.  NULL means 0.
 *   h0, last_state   : (batch, dim, dstate) fp32, contiguous.  h0 NULL means a
 *                      zero initial state; last_state NULL means "not wanted".
 *   z NULL           : no gate (out = y).
 *   delta_softplus   : nonzero applies softplus to delta + bias.
 * Sizes: batch, dim, seqlen >= 0 (zero sizes are a no-op, except that
 * seqlen == 0 with last_state set copies h0, or zeros, into last_state);
 * 1 <= dstate <= SSM_MAX_DSTATE; ngroups (0 or 1 meaning one group) must
 * divide dim; seqlen must be below 2^31 - 64.  The kernel reads each group
 * of 4 channels, and the state rows of B and C, through 32-bit byte
 * windows: (3 * dim_stride + seqlen) * element size for u, delta, z and out,
 * and (r * group_stride + (dstate - 1) * state_stride + seqlen) * element
 * size for B and C, must stay below 2^32, with r = 0 when dim / ngroups is
 * a multiple of 16 (or one group) and min(3, ngroups - 1) otherwise; with
 * checkpoints, 4 * ceil(seqlen / 16) * dstate * 4 bytes too.  Larger spans
 * return SSM_ERR_UNSUPPORTED.
 * Aliasing: out must not overlap u, delta, z, B or C; last_state must not
 * overlap any input except that it may be exactly h0 (in-place carry).
 * Workspace: device scratch owned by the caller, 4-byte aligned, of at least
 * ssm_scan_workspace_size() bytes, not overlapping any tensor.  The library
 * uses it to cut long sequences with few channels into segments scanned in
 * parallel; with workspace NULL or too small the scan still runs, correctly,
 * as a single segment per sequence.  Its contents are scratch on return.
 * Checkpoints (optional output, for ssm_selective_scan_bwd): fp32
 * (batch, dim, ceil(seqlen / SSM_CHECKPOINT_TOKENS), dstate), contiguous;
 * element (b, d, k, n) is the state h[n] entering token
 * k * SSM_CHECKPOINT_TOKENS (so k = 0 holds h0, or zeros).  NULL: none
 * written.  Must not overlap any other tensor.
 * Fused conv branch (Mamba model notes, section 4.3: the branch that feeds
 * the SSM first passes a local causal convolution).  With conv_weight set,
 * `u` is the conv input x and the SSM input is computed per token as
 *     u_t = act(conv_bias[d] + sum_{k<d_conv} conv_weight[d,k] x_{t-(d_conv-1)+k})
 * with act = SiLU when conv_silu is nonzero, else identity:
 *   conv_weight     : (dim, d_conv) fp32, contiguous; 1 <= d_conv <= SSM_MAX_CONV.
 *   conv_bias       : (dim) fp32; NULL means 0.
 *   conv_state_in   : (batch, dim, d_conv) fp32, contiguous, holding the inputs
 *                     before the sequence (element k = x_{k-d_conv}); NULL
 *                     means zeros.
 *   conv_state_out  : same layout, receives the last d_conv inputs
 *                     x_{seqlen-d_conv} .. x_{seqlen-1} (from conv_state_in
 *                     where seqlen < d_conv); NULL: not wanted.  It is the
 *                     conv_state the decode update continues from.
 *   conv_out        : (batch, dim, seqlen), io_dtype, time stride 1: receives
 *                     the SSM input u (e.g. for the backward); NULL: not wanted.
 *   None of them may overlap any other tensor. */
typedef struct ssm_scan_args {
  int64_t batch, dim, seqlen, dstate;
  int32_t io_dtype;       /* ssm_dtype */
  int32_t delta_softplus; /* bool */
  const void* u;      int64_t u_batch_stride, u_dim_stride;
  const void* delta;  int64_t delta_batch_stride, delta_dim_stride;
  const void* z;      int64_t z_batch_stride, z_dim_stride;
  const void* B;      int64_t B_batch_stride, B_state_stride;
  const void* C;      int64_t C_batch_stride, C_state_stride;
  const float* A;     int64_t A_dim_stride, A_state_stride;
  const float* D;
  const float* delta_bias;
  const float* h0;
  float* last_state;
  void* out;          int64_t out_batch_stride, out_dim_stride;
  void* workspace;    size_t workspace_bytes;
  float* checkpoints;
  const float* conv_weight;
  const float* conv_bias;
  const float* conv_state_in;
  float* conv_state_out;
  void* conv_out;     int64_t conv_out_batch_stride, conv_out_dim_stride;
  int32_t d_conv;
  int32_t conv_silu;  /* bool */
  int64_t ngroups;    /* B/C groups; 0 or 1: one group */
  int64_t B_group_stride, C_group_stride;
} ssm_scan_args;

/* Arguments of the scan backward.  The forward inputs (u, delta, z, B, C, A,
 * D, delta_bias, h0, delta_softplus) keep their meaning, layout and strides
 * from ssm_scan_args and must be the ones the forward ran with;
 * `checkpoints` (required) is what that forward wrote.
 *   dout            : (batch, dim, seqlen), io_dtype, time stride 1: the
 *                     gradient on out.
 *   dlast           : (batch, dim, dstate) fp32, contiguous: the gradient on
 *                     last_state.  NULL means 0.
 * Outputs (device memory owned by the caller, fully overwritten):
 *   du, ddelta      : (batch, dim, seqlen), io_dtype, time stride 1.
 *   dz              : the same, required when z is given, else ignored.
 *   dB, dC          : (batch, ngroups, dstate, seqlen) fp32, contiguous
 *                     (each summed over the channels of its group).
 *   dA              : (dim, dstate) fp32, contiguous (summed over batch, time).
 *   dD, ddelta_bias : (dim) fp32 (summed over batch, time); NULL: not wanted.
 *   dh0             : (batch, dim, dstate) fp32, contiguous; NULL: not wanted.
 * The sums over channels (dB, dC) and over batch rows (dA, dD, ddelta_bias)
 * are accumulated with device atomics when no workspace is given, so their
 * last bits can vary from run to run; with a workspace every output is
 * deterministic.  Outputs must not overlap
 * each other or any input.  With the workspace, long sequences with few
 * channels are cut into segments: a pass over segments 1..G-1 records the
 * adjoint leaving each segment at its start (the adjoint recurrence needs no
 * forward state), and every segment then runs the full backward from the
 * exact adjoint entering it (Mamba paper notes, section 5.4: state passed at
 * chunk edges); without it, each sequence is one segment.
 * It is built for dstate 1..SSM_MAX_DSTATE and for B/C groups that keep each
 * block of 16 consecutive channels in one group (one group, or dim / ngroups
 * a multiple of 16); other groupings return SSM_ERR_UNSUPPORTED.
 * Workspace (optional): device scratch owned by the caller, 4-byte aligned,
 * of at least ssm_scan_bwd_workspace_size() bytes, not overlapping any
 * tensor.  The library then writes each block of 16 channels' dB/dC partial
 * sums, and each segment's and batch row's dA, dD and ddelta_bias, there with plain
 * stores and adds them in fixed order in second passes, instead of adding
 * into the outputs with device atomics: every output is then deterministic,
 * and the time no longer depends on where dB and dC sit (the atomics on
 * dB(n, t) and dC(n, t) are issued together and at some offsets between the
 * two buffers share memory channels).  With workspace NULL or too small the
 * atomics are used.
 * Its contents are scratch on return. */
typedef struct ssm_scan_bwd_args {
  int64_t batch, dim, seqlen, dstate;
  int32_t io_dtype;       /* ssm_dtype */
  int32_t delta_softplus; /* bool */
  const void* u;      int64_t u_batch_stride, u_dim_stride;
  const void* delta;  int64_t delta_batch_stride, delta_dim_stride;
  const void* z;      int64_t z_batch_stride, z_dim_stride;
  const void* B;      int64_t B_batch_stride, B_state_stride;
  const void* C;      int64_t C_batch_stride, C_state_stride;
  const float* A;     int64_t A_dim_stride, A_state_stride;
  const float* D;
  const float* delta_bias;
  const float* h0;
  const float* checkpoints;
  const void* dout;   int64_t dout_batch_stride, dout_dim_stride;
  const float* dlast;
  void* du;           int64_t du_batch_stride, du_dim_stride;
  void* ddelta;       int64_t ddelta_batch_stride, ddelta_dim_stride;
  void* dz;           int64_t dz_batch_stride, dz_dim_stride;
  float* dB;
  float* dC;
  float* dA;
  float* dD;
  float* ddelta_bias;
  float* dh0;
  int64_t ngroups;    /* B/C groups; 0 or 1: one group */
  int64_t B_group_stride, C_group_stride;
  void* workspace;    size_t workspace_bytes;
} ssm_scan_bwd_args;

/* Arguments of the single-token decode update.
 *   state            : (batch, dim, dstate) fp32, state stride 1, element
 *                      (b, d, n) at state[b * state_batch_stride +
 *                      d * state_dim_stride + n]; updated IN PLACE.
 *   x, dt, z, out    : (batch, dim), dim stride 1.  z NULL means no gate.
 *   B, C             : (batch, ngroups, dstate), state stride 1; element
 *                      (b, g, n) at ptr[b * *_batch_stride + g * *_group_stride
 *                      + n]; channel d reads group d / (dim / ngroups).
 *   A                : (dim, dstate) fp32, state stride 1.
 *   D, dt_bias       : (dim) fp32, contiguous, NULL means 0.
 * Fused conv branch (as in ssm_scan_args): with conv_weight set, x is the
 * conv input; conv_state (batch, dim, d_conv) fp32, contiguous, holds the
 * previous d_conv inputs and is shifted in place (oldest dropped, x appended);
 * the SSM input is act(conv_bias + sum_k conv_weight[d,k] conv_state[k]) of
 * the updated conv_state.  1 <= d_conv <= SSM_MAX_CONV.
 * Sizes: batch, dim >= 0 (zero is a no-op); 1 <= dstate <= SSM_MAX_DSTATE;
 * ngroups (0 or 1 meaning one group) must divide dim; batch at most 65535.
 * Aliasing: out must not overlap state or any input; state and conv_state
 * must not overlap any input or each other. */
typedef struct ssm_update_args {
  int64_t batch, dim, dstate;
  int32_t io_dtype;    /* ssm_dtype */
  int32_t dt_softplus; /* bool */
  float* state;       int64_t state_batch_stride, state_dim_stride;
  const void* x;      int64_t x_batch_stride;
  const void* dt;     int64_t dt_batch_stride;
  const void* z;      int64_t z_batch_stride;
  const void* B;      int64_t B_batch_stride;
  const void* C;      int64_t C_batch_stride;
  const float* A;     int64_t A_dim_stride;
  const float* D;
  const float* dt_bias;
  void* out;          int64_t out_batch_stride;
  float* conv_state;
  const float* conv_weight;
  const float* conv_bias;
  int32_t d_conv;
  int32_t conv_silu;  /* bool */
  int64_t ngroups;    /* B/C groups; 0 or 1: one group */
  int64_t B_group_stride, C_group_stride;
} ssm_update_args;

/* Arguments of the Mamba-2 SSM (the SSD layer) prefill.  The Mamba-2
 * section of the mamba_ssm notes and the skill page's Mamba-2 configuration
 * make the block multi-head (nheads heads of headdim channels, ngroups B/C
 * groups), and its printed parameter count has one A, one D and one step bias
 * per head.  For batch row b, head h (reading B/C group g = h / (nheads /
 * ngroups)), head channel p and state n:
 *     Delta_t  = softplus(dt[b,t,h] + dt_bias[h])      (identity without softplus)
 *     S_t[p,n] = exp(Delta_t * A[h]) * S_{t-1}[p,n] + Delta_t * B[b,t,g,n] * x[b,t,h,p]
 *     out[b,t,h,p] = (sum_n C[b,t,g,n] * S_t[p,n] + D[h] * x[b,t,h,p]) * silu(z[b,t,h,p])
 * from S_{-1} = h0[b,h] (or zero), optionally returning S_{L-1}.  The kernel
 * evaluates it in chunks of 64 tokens through the equivalent structured
 * matrix form (state space duality) on the matrix cores.
 *   x, z, out   : (batch, seqlen, nheads, headdim), headdim stride 1;
 *                 element (b, t, h, p) at ptr[b * *_batch_stride +
 *                 t * *_seq_stride + h * *_head_stride + p].
 *   dt          : (batch, seqlen, nheads), head stride 1, io_dtype.
 *   B, C        : (batch, seqlen, ngroups, dstate), state stride 1.
 *   A, D, dt_bias : (nheads) fp32; D and dt_bias NULL mean 0.
 *   h0, last_state : (batch, nheads, headdim, dstate) fp32, contiguous; h0
 *                 NULL is a zero initial state, last_state NULL: not wanted.
 *   z NULL      : no gate.
 * Sizes: batch, seqlen >= 0 (zero is a no-op; seqlen 0 with last_state
 * copies h0, or zeros); nheads, headdim, dstate >= 1; ngroups 0 or 1 (one
 * group) or a divisor of nheads; seqlen below 2^31 - 64; dstate at most 128
 * for bf16 IO and 64 for fp32 IO (SSM_ERR_UNSUPPORTED past that); batch *
 * nheads * ceil(headdim / 16) below 2^31.  The kernel reaches 64 tokens of a
 * (batch, head) slice of x, z, dt and out and of a (batch, group) slice of B
 * and C through 31-bit byte windows: (63 * seq_stride + inner size) * element
 * size must stay below 2^31 (inner size headdim, 1 for dt, dstate for B/C);
 * larger strides return SSM_ERR_UNSUPPORTED.
 * Precision: fp32 accumulation throughout and an fp32 state.  With bf16 IO the
 * products run on bf16 operands, so the masked chunk scores and x weighted
 * by the decays are rounded to bf16 where they enter a product, and the fp32
 * state entering each chunk enters as a bf16 value plus its bf16 remainder
 * (two products); with fp32 IO every product is fp32.
 * Aliasing: out must not overlap any input; last_state must not overlap any
 * input except that it may be exactly h0.
 * Workspace: device scratch owned by the caller, 4-byte aligned, of at least
 * ssm_ssd_workspace_size() bytes, not overlapping any tensor.  With it, a
 * long sequence whose (batch, head) slices alone would leave the GPU idle is
 * cut into segments scanned in parallel (Mamba paper notes, sections
 * 5.3/5.4: chunks handing the state on), the state entering each segment
 * folded from the end states of the earlier ones; the result is the
 * one-segment result up to fp32 rounding.  With workspace NULL or too small
 * each sequence is one segment.  Its contents are scratch on return. */
typedef struct ssm_ssd_args {
  int64_t batch, seqlen, nheads, headdim, ngroups, dstate;
  int32_t io_dtype;      /* ssm_dtype */
  int32_t dt_softplus;   /* bool */
  const void* x;   int64_t x_batch_stride, x_seq_stride, x_head_stride;
  const void* dt;  int64_t dt_batch_stride, dt_seq_stride;
  const void* z;   int64_t z_batch_stride, z_seq_stride, z_head_stride;
  const void* B;   int64_t B_batch_stride, B_seq_stride, B_group_stride;
  const void* C;   int64_t C_batch_stride, C_seq_stride, C_group_stride;
  const float* A;
  const float* D;
  const float* dt_bias;
  const float* h0;
  float* last_state;
  void* out;       int64_t out_batch_stride, out_seq_stride, out_head_stride;
  void* workspace;    size_t workspace_bytes;
} ssm_ssd_args;

/* ABI version of the loaded library (SSM_ABI_VERSION at build time). */
int ssm_abi_version(void);

/* sizeof the argument structs, for bindings that mirror them. */
size_t ssm_scan_args_size(void);
size_t ssm_scan_bwd_args_size(void);
size_t ssm_update_args_size(void);
size_t ssm_ssd_args_size(void);

/* Workspace bytes the scan can use for this argument block (0 when it would
 * run single-segment anyway): for G segments, with BD = batch * dim and
 * each part rounded up to 256 bytes, the segment aggregates BD * G *
 * (dstate + 1) floats, the records of the 10 windows of each segment's
 * head BD * G * 10 * (dstate + 1) floats, and BD * G * 21 ints of work
 * lists.  Reads only sizes; pure host code. */
size_t ssm_scan_workspace_size(const ssm_scan_args* args);

/* Workspace bytes the SSD prefill can use for this argument block (0 when
 * it would run as one segment anyway): for G segments, the segment end
 * states batch * nheads * G * headdim * dstate fp32 values (rounded up to
 * 256 bytes) and their step-size sums, batch * nheads * G more.  Reads only
 * sizes; pure host code. */
size_t ssm_ssd_workspace_size(const ssm_ssd_args* args);

/* Workspace bytes the backward can use for this argument block:
 * batch * ceil(dim / 16) * 2 * dstate * seqlen + G * batch * dim *
 * (dstate + 2) fp32 values, plus batch * dim * G * (dstate + 1) for the
 * adjoint aggregates when the sequence is cut into G > 1 segments (0 for an empty
 * sequence or when batch * ngroups exceeds 65535, where it adds dB/dC with
 * atomics anyway).  Reads only sizes; pure host code. */
size_t ssm_scan_bwd_workspace_size(const ssm_scan_bwd_args* args);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* ssm_status_string(int status);

/* Pure host checks of an argument block: no HIP call, no device access, so
 * they run on a machine without a GPU.  Returns the first failing status. */
int ssm_validate_scan(const ssm_scan_args* args);
int ssm_validate_scan_bwd(const ssm_scan_bwd_args* args);
int ssm_validate_update(const ssm_update_args* args);
int ssm_validate_ssd(const ssm_ssd_args* args);

/* Prefill scan (see ssm_scan_args).  Validates, then launches on `stream`. */
int ssm_selective_scan_fwd(const ssm_scan_args* args, void* stream);

/* The prefill scan for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels as ssm_selective_scan_fwd, and it calls no
 * allocating routine.  args->workspace and args->workspace_bytes are ignored;
 * long sequences with few channels are cut into segments with their
 * aggregates, window records and work lists kept in a static device buffer
 * of SSM_NOALLOC_SCRATCH_BYTES that the library holds on every device it
 * runs on until the process ends (its address is looked up on the first
 * call on each device).  That is enough for every argument block with
 * dstate <= 16 (at most 17 MB are needed); with more states, blocks whose
 * segment scratch, ssm_scan_workspace_size(args) bytes, exceeds it return
 * SSM_ERR_SCRATCH and launch nothing.  Every call on
 * a device shares that device's buffer: calls on one device that may
 * overlap in time (different streams, no ordering between them) race on it
 * and must be serialised by the caller.  The buffer holds no state between
 * calls that needs clearing.  Returns an ssm_status. */
int ssm_selective_scan_fwd_noalloc(const ssm_scan_args* args, void* stream);

/* Scan backward (see ssm_scan_bwd_args).  Validates, then launches on
 * `stream`. */
int ssm_selective_scan_bwd(const ssm_scan_bwd_args* args, void* stream);

/* Decode update (see ssm_update_args).  Validates, then launches on `stream`. */
int ssm_selective_state_update(const ssm_update_args* args, void* stream);

/* Mamba-2 SSM prefill (see ssm_ssd_args).  Validates, then launches on
 * `stream`. */
int ssm_ssd_scan_fwd(const ssm_ssd_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H_ */
