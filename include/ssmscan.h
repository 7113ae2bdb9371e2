/*
 * ssmscan.h -- C ABI of libssmscan.so: the Mamba selective-scan forward
 * operator and its width-4 causal depthwise conv prologue, for AMD MI355X
 * (gfx950).
 *
 * Operation (PaddleNLP Kernel operator-library guide, section 4.1
 * "selective_scan": selective_scan_fn(u, delta, A, B, C, D, z, delta_bias,
 * delta_softplus, return_last_state)).  For every batch b, channel d and
 * state s, with delta' = softplus(delta + delta_bias) when delta_softplus is
 * set (otherwise delta + delta_bias):
 *
 *     x_t[s] = exp(delta'_t * A[d,s]) * x_{t-1}[s] + delta'_t * B_t[s] * u_t
 *     y_t    = sum_s C_t[s] * x_t[s]
 *     out_t  = (y_t + D[d] * u_t) * silu(z_t)          (D, z optional)
 *     last_state[b,d,s] = x_{seqlen-1}[s]              (optional)
 *
 * with x_{-1} = initial_state (zero when not given).  The recurrence is not
 * printed on the pages; it is the standard zero-order-hold discretisation.
 *
 * Shapes (same section): u, delta, z, out: (batch, dim, seqlen); A: (dim,
 * dstate), real; B and C each either fixed (dim, dstate) or time-varying
 * grouped (batch, ngroups, dstate, seqlen) -- the page's 3-D (batch, dstate,
 * seqlen) form is ngroups = 1; D, delta_bias: (dim,); last_state and
 * initial_state: (batch, dim, dstate).  Grouped channel d uses group
 * d / (dim / ngroups).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers to dense row-major tensors (innermost
 *    stride 1).  The caller owns and allocates every buffer, including the
 *    outputs.  `out` must not alias an input.
 *  - "io" tensors (u, delta, z, B, C, out, conv x) all have the dtype
 *    io_dtype: SSM_F32 (IEEE binary32), SSM_BF16 (bfloat16, stored as the
 *    upper 16 bits of a binary32) or SSM_F16 (IEEE binary16).  A, D, delta_bias, conv weight and bias,
 *    initial_state and last_state are always binary32; the state is binary32.
 *    bf16 and fp16 outputs are rounded to nearest, ties to even.
 *  - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL is
 *    the default stream).  Nothing synchronises.
 *  - Errors: arguments are checked on the host before anything is enqueued.
 *    Status 1-3 and 5 leave all memory untouched.  Status 4 means a HIP call
 *    failed while enqueueing (ssm_last_hip_error() gives the hipError_t).
 *  - The library allocates no memory and reads no environment variables: the
 *    caller passes every buffer, scratch included (the *_workspace_size
 *    queries give the size).  It keeps no state between calls except a
 *    cached device property query; calls from several host threads are safe.
 */
#ifndef SSMSCAN_H
#define SSMSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 13
#define SSM_CKPT_INTERVAL 32  /* timesteps between saved states (checkpoints) */
#define SSM_MAX_DSTATE 16   /* largest dstate the kernels are built for */
#define SSM_CONV_WIDTH 4    /* the one conv width the kernels are built for */
#define SSM_NOALLOC_SCRATCH_BYTES (8u << 20)   /* built-in scratch of ssm_scan_fwd_noalloc, per device */

/* io dtype.  SSM_F16 (IEEE binary16) is taken by every entry point except
 * ssd_scan_fwd (bf16 only), which returns SSM_ERR_UNSUPPORTED for it. */
enum { SSM_F32 = 0, SSM_BF16 = 1, SSM_F16 = 2 };
/* layout of B and C (one kind per tensor) */
enum { SSM_BC_FIXED = 0,    /* (dim, dstate) */
       SSM_BC_VARYING = 1   /* (batch, ngroups, dstate, seqlen) */ };
/* conv activation ("swish" on the page is silu) */
enum { SSM_ACT_NONE = 0, SSM_ACT_SILU = 1 };
/* status codes */
enum {
  SSM_OK = 0,
  SSM_ERR_NULL = 1,         /* a required pointer is NULL */
  SSM_ERR_SHAPE = 2,        /* a size <= 0, dim % ngroups != 0, or overflow */
  SSM_ERR_UNSUPPORTED = 3,  /* dtype, dstate > 16, conv width != 4, bad enum */
  SSM_ERR_HIP = 4,          /* a HIP runtime call failed */
  SSM_ERR_WORKSPACE = 5,    /* scratch needed but workspace NULL or too small */
  SSM_ERR_SCRATCH = 6       /* ssm_scan_fwd_noalloc: the plan needs more than its scratch */
};

/* Arguments of ssm_scan_fwd.  Every pointer is a device pointer. */
typedef struct ssm_scan_args {
  int64_t batch, dim, seqlen, dstate, ngroups;  /* ngroups: 1 unless grouped */
  int32_t io_dtype;                             /* SSM_F32 or SSM_BF16 */
  const void *u;                                /* (b,d,l) io; ignored with conv */
  const void *delta;                            /* (b,d,l) io, required */
  const float *A;                               /* (d,n) fp32, required */
  const void *B; int32_t B_kind;                /* io, SSM_BC_* */
  const void *C; int32_t C_kind;                /* io, SSM_BC_* */
  const float *D;                               /* (d) fp32 or NULL */
  const float *delta_bias;                      /* (d) fp32 or NULL */
  const void *z;                                /* (b,d,l) io or NULL */
  int32_t delta_softplus;                       /* 0 or 1 */
  void *out;                                    /* (b,d,l) io, required */
  float *last_state;                            /* (b,d,n) fp32 or NULL */
  const float *initial_state;                   /* (b,d,n) fp32 or NULL (zero) */
  /* Optional fused conv prologue (same page, section 4.2 causal_conv1d):
   * when conv_weight != NULL, u is not read and is replaced by
   *   u = round_io(act(conv_bias[d] + sum_k conv_weight[d,k] * conv_x[b,d,t-3+k]))
   * with conv_x[t<0] = 0 -- exactly what causal_conv1d_fwd stores. */
  const void *conv_x;                           /* (b,d,l) io */
  const float *conv_weight;                     /* (d, conv_width) fp32 */
  const float *conv_bias;                       /* (d) fp32 or NULL */
  int32_t conv_width;                           /* must be 4 */
  int32_t conv_act;                             /* SSM_ACT_* */
  /* Scratch for the sequence-split plan (see ssm_scan_workspace_size),
   * caller-allocated device memory of workspace_bytes bytes.  The library
   * allocates nothing: when the plan needs scratch and workspace is NULL or
   * smaller than ssm_scan_workspace_size reports, the call returns
   * SSM_ERR_WORKSPACE before anything is enqueued.  It is not read before it
   * is written, so it needs no clearing, and it may be reused once the call's
   * work on hip_stream has finished. */
  void *workspace;
  size_t workspace_bytes;
  /* Optional output for the backward (ssm_scan_bwd): the state before every
   * SSM_CKPT_INTERVAL-th timestep, (batch, dim, nck, dstate) fp32 with
   * nck = ceil(seqlen / SSM_CKPT_INTERVAL); entry k is x_{k*32-1}, so entry 0
   * is initial_state (zero when not given).  NULL: not written. */
  float *checkpoints;
  /* Sequence split: 0 lets the library choose its plan (it splits the
   * sequence only when the channels alone leave the GPU short of waves, and
   * at dstate 13..16 may run leftover channels with eight lanes per channel
   * to even out the load per SIMD); k >= 1 asks for k segments (equal
   * lengths of whole chunks, so possibly fewer) of the four-lane kernel.
   * The plan changes the results only by rounding order.  Negative values
   * return SSM_ERR_SHAPE. */
  int32_t seq_segments;
} ssm_scan_args_t;

/* Selective-scan forward.  Enqueues the scan on hip_stream and returns a
 * status code (SSM_OK on success). */
int ssm_scan_fwd(const ssm_scan_args_t *args, void *hip_stream);

/* ssm_scan_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and status codes as ssm_scan_fwd, except that
 * args->workspace and workspace_bytes are ignored: the scratch of the plan
 * (the sequence segments' end states) lives in a buffer built into the
 * library, SSM_NOALLOC_SCRATCH_BYTES per device, held until the process
 * ends.  A plan that needs more scratch than that returns SSM_ERR_SCRATCH
 * before anything is enqueued (ssm_scan_workspace_size gives the need; the
 * Mamba-shaped layers need at most 6.6 MiB).  The caller still allocates
 * every input and output.  The call allocates nothing: the first call on a
 * device looks the buffer's address up once (hipGetSymbolAddress).  Every
 * call on one device shares that device's buffer and leaves its contents
 * behind, so calls that overlap on one device -- different streams, or
 * different threads -- race and give wrong results; calls ordered on one
 * stream are safe. */
int ssm_scan_fwd_noalloc(const ssm_scan_args_t *args, void *hip_stream);

/* Host-only argument check of ssm_scan_fwd: the same status the call would
 * return before enqueueing anything.  Touches no device memory and makes no
 * HIP call, so it is usable on a machine without a GPU. */
int ssm_scan_validate(const ssm_scan_args_t *args);

/* Scratch bytes ssm_scan_fwd needs for these arguments (0 when the plan keeps
 * the whole sequence in one pass).  Host-only: no HIP call except cached
 * queries of the device's compute-unit count and of how many workgroups of
 * a kernel one compute unit holds (on a machine without a GPU those fail and
 * the plan assumes 256 compute units and no mixed plan). */
int ssm_scan_workspace_size(const ssm_scan_args_t *args, size_t *bytes);

/* The launch plan ssm_scan_fwd takes for these arguments (same queries as
 * ssm_scan_workspace_size).  Every wave runs lanes_per_channel lanes per
 * channel over 64 / lanes_per_channel channels; at dstate 13..16 the mixed
 * plan runs the channel blocks left over after whole waves fill the SIMDs
 * evenly as eight_lane_waves waves of eight lanes per channel (8 channels,
 * about half the work each). */
typedef struct {
  int32_t segments;            /* sequence segments (1: one pass) */
  int32_t waves;               /* waves of lanes_per_channel lanes, per segment */
  int32_t lanes_per_channel;
  int32_t eight_lane_waves;    /* mixed plan's extra waves (0: not mixed) */
  size_t workspace_bytes;      /* as ssm_scan_workspace_size */
} ssm_scan_plan_t;
int ssm_scan_plan(const ssm_scan_args_t *args, ssm_scan_plan_t *plan);

/* Selective-scan forward with complex A (the same page, section 4.1: A
 * (dim, dstate) may be real or complex; nothing more is printed about the
 * complex case).  Read as the recurrence above over the complex numbers, with
 * B and C complex too (a real B or C is the case of zero imaginary parts),
 * and the output the real part of the contraction:
 *
 *     x_t[s] = exp(delta'_t A[d,s]) x_{t-1}[s] + delta'_t B_t[s] u_t   (complex)
 *     y_t    = Re(sum_s C_t[s] x_t[s]),   out_t = (y_t + D[d] u_t) silu(z_t)
 *
 * delta', u, z, D, delta_bias and out are real as in ssm_scan_fwd.  The
 * arguments are those of ssm_scan_fwd with these layouts, every complex value
 * a (real, imaginary) pair with the pair innermost:
 *   A: (dim, dstate, 2) fp32;
 *   B, C: io, fixed (dim, dstate, 2) or varying (batch, ngroups, dstate,
 *         seqlen, 2);
 *   initial_state, last_state: (batch, dim, dstate, 2) fp32 or NULL;
 *   checkpoints: (batch, dim, nck, dstate, 2) fp32 or NULL, the state before
 *         every SSM_CKPT_INTERVAL-th timestep, for ssm_scan_bwd_complex.
 * Not taken (SSM_ERR_UNSUPPORTED): the fused conv prologue (conv_weight must
 * be NULL; run causal_conv1d_fwd first).  u is required; workspace is ignored
 * (the sequence is walked in one pass).  The decay's phase uses the
 * hardware sine and cosine on the fractional part of delta' Im(A) / (2 pi),
 * and delta' is the softplus without the cancellation of 1 + e^v (a large
 * |Im A| magnifies an error in delta').  Same conventions and status codes
 * as ssm_scan_fwd. */
int ssm_scan_fwd_complex(const ssm_scan_args_t *args, void *hip_stream);

/* Host-only argument check of ssm_scan_fwd_complex (no HIP call). */
int ssm_scan_complex_validate(const ssm_scan_args_t *args);

/* Arguments of ssm_scan_bwd.  Every pointer is a device pointer.  The inputs
 * are those of the forward call (same shapes, dtypes and layout kinds);
 * checkpoints are the ones that forward call wrote. */
typedef struct ssm_scan_bwd_args {
  int64_t batch, dim, seqlen, dstate, ngroups;
  int32_t io_dtype;
  const void *u;                                /* (b,d,l) io, required */
  const void *delta;                            /* (b,d,l) io, required */
  const float *A;                               /* (d,n) fp32, required */
  const void *B; int32_t B_kind;                /* io, SSM_BC_* */
  const void *C; int32_t C_kind;                /* io, SSM_BC_* */
  const float *D;                               /* (d) fp32 or NULL */
  const float *delta_bias;                      /* (d) fp32 or NULL */
  const void *z;                                /* (b,d,l) io or NULL */
  int32_t delta_softplus;                       /* 0 or 1 */
  const float *checkpoints;                     /* (b,d,nck,n) fp32 from ssm_scan_fwd, required */
  const void *dout;                             /* (b,d,l) io: dL/d out, required */
  /* gradients, caller-allocated and fully overwritten */
  void *du;                                     /* (b,d,l) io, required */
  void *ddelta;                                 /* (b,d,l) io, required */
  void *dz;                                     /* (b,d,l) io, required iff z */
  float *dA;                                    /* (d,n) fp32, required */
  float *dB;                                    /* fp32, B's layout ((d,n) or (b,g,n,l)), required */
  float *dC;                                    /* fp32, C's layout, required */
  float *dD;                                    /* (d) fp32, required iff D */
  float *ddelta_bias;                           /* (d) fp32, required iff delta_bias */
  float *dinitial_state;                        /* (b,d,n) fp32 or NULL */
  /* Scratch for the per-workgroup partial sums (ssm_scan_bwd_workspace_size),
   * caller-allocated device memory; the library allocates nothing, and a NULL
   * or too small workspace returns SSM_ERR_WORKSPACE before anything is
   * enqueued.  Every partial is written before it is read. */
  void *workspace;
  size_t workspace_bytes;
  /* Sequence split: 0 lets the library choose how many segments of whole
   * SSM_CKPT_INTERVAL chunks the sequence is cut into (it splits when the
   * channels alone leave compute units idle); k >= 1 asks for at most k
   * segments (equal whole-chunk lengths, so possibly fewer).  Segments after
   * the first first get their adjoint carry from a pass of their own; the
   * results differ from the unsplit ones only by rounding order.  Negative
   * values return SSM_ERR_SHAPE. */
  int32_t seq_segments;
} ssm_scan_bwd_args_t;

/* Selective-scan backward (the same page, section 4.1: the operator's
 * backward is the extension's bwd entry; last_state carries no gradient).
 * Given dout = dL/d out, writes the gradient of L with respect to every input
 * of the forward:  with h_t = dL/dx_t, the adjoint of the recurrence,
 *
 *     g_t     = dout_t * silu(z_t)                     (dL/d(y_t + D u_t))
 *     h_t[s]  = g_t * C_t[s] + exp(delta'_{t+1} A[d,s]) * h_{t+1}[s],  h_l = 0
 *     du_t    = g_t D[d] + delta'_t sum_s h_t[s] B_t[s]
 *     ddelta_t = softplus'(delta_t + delta_bias[d]) *
 *                sum_s h_t[s] (A[d,s] exp(delta'_t A[d,s]) x_{t-1}[s] + B_t[s] u_t)
 *     dA[d,s] = sum_{b,t} h_t[s] delta'_t exp(delta'_t A[d,s]) x_{t-1}[s]
 *     dB_t[s] = sum over the group's channels of h_t[s] delta'_t u_t   (fixed: summed over b, t)
 *     dC_t[s] = sum over the group's channels of g_t x_t[s]           (fixed: summed over b, t)
 *     dD[d]   = sum_{b,t} g_t u_t,   ddelta_bias[d] = sum_{b,t} ddelta_t
 *     dz_t    = dout_t (y_t + D u_t) silu'(z_t),  dinitial_state = exp(delta'_0 A) h_0
 *
 * (softplus' = 1 without delta_softplus).  Every chunk of SSM_CKPT_INTERVAL
 * timesteps is re-run forward from its checkpoint, then walked in reverse.
 * Every sum over channels, batches and timesteps is taken in a fixed order,
 * so results are bit-for-bit repeatable.  Same conventions and status codes
 * as ssm_scan_fwd. */
int ssm_scan_bwd(const ssm_scan_bwd_args_t *args, void *hip_stream);

/* Gradients of the complex-A forward (ssm_scan_fwd_complex; the same page,
 * section 4.1: A may be complex, and the operator has a backward).  The
 * arguments are those of ssm_scan_bwd read with the complex forward's
 * layouts: A (d,n,2) fp32; B/C io pairs, (d,n,2) fixed or (b,g,n,l,2)
 * varying; checkpoints (b,d,nck,n,2) fp32 written by ssm_scan_fwd_complex;
 * dA (d,n,2), dB/dC in B's/C's pair layout and dinitial_state (b,d,n,2),
 * all fp32, each the gradient of the real and of the imaginary part
 * (G_v = dL/dRe v + i dL/dIm v).  With a_t = exp(delta'_t A):
 *
 *     h_t     = dy_t conj(C_t) + conj(a_{t+1}) h_{t+1},  h_l = 0
 *     dC_t    = dy_t conj(x_t),   G_a = h_t conj(x_{t-1})
 *     dA     += conj(delta'_t a_t) G_a,   dB_t = delta'_t u_t h_t
 *     du_t    = D dy_t + delta'_t sum_s Re(h_t conj(B_t))
 *     ddelta_t = softplus'(.) (sum_s Re(G_a conj(A a_t)) + u_t sum_s Re(h_t conj(B_t)))
 *
 * with dy, dz, dD and d(delta_bias) as in ssm_scan_bwd.  delta'_t is formed
 * as in ssm_scan_fwd_complex, and the phase of a_t to about one rounding
 * (Im(A) / (2 pi) held as two floats, the product's rounding error
 * recovered with an fma): ddelta weighs a phase error by |A|^2 delta'.
 * seq_segments splits the sequence as in ssm_scan_bwd (0: the library's
 * choice, k >= 1: at most k segments of whole chunks): a carry pass walks
 * every segment after the first from a zero carry, and each segment starts
 * from the carry of the later ones, the same recurrence reassociated (the
 * decay over a segment is the product of its a_t, multiplied up step by
 * step).  The
 * workspace (ssm_scan_bwd_complex_workspace_size) holds the partial sums and
 * the carries and is required.  Asynchronous on hip_stream; returns a status
 * code. */
int ssm_scan_bwd_complex(const ssm_scan_bwd_args_t *args, void *hip_stream);

/* Host-only argument check of ssm_scan_bwd_complex (no HIP call). */
int ssm_scan_bwd_complex_validate(const ssm_scan_bwd_args_t *args);

/* Scratch bytes ssm_scan_bwd_complex needs (no HIP call). */
int ssm_scan_bwd_complex_workspace_size(const ssm_scan_bwd_args_t *args, size_t *bytes);

/* Host-only argument check of ssm_scan_bwd (no HIP call). */
int ssm_scan_bwd_validate(const ssm_scan_bwd_args_t *args);

/* Scratch bytes ssm_scan_bwd needs for these arguments.  Host-only, no HIP
 * call except a cached query of the device's compute-unit count. */
int ssm_scan_bwd_workspace_size(const ssm_scan_bwd_args_t *args, size_t *bytes);

/* Causal depthwise conv forward (PaddleNLP Kernel operator-library guide,
 * section 4.2 "causal_conv1d": causal_conv1d_fn(x, weight, bias, ...,
 * activation)).  x, out: (batch, dim, seqlen) io, device pointers; weight:
 * (dim, width) fp32; bias: (dim) fp32 or NULL; act: SSM_ACT_NONE or
 * SSM_ACT_SILU.
 *   out[b,d,t] = round_io(act(bias[d] + sum_k weight[d,k] * x[b,d,t-(width-1)+k]))
 * with x[t<0] = 0 (cross-correlation with left zero padding).  width must be
 * 4.  Asynchronous on hip_stream; returns a status code. */
int causal_conv1d_fwd(const void *x, const float *weight, const float *bias, void *out,
                      int64_t batch, int64_t dim, int64_t seqlen, int32_t width,
                      int32_t io_dtype, int32_t act, void *hip_stream);

/* causal_conv1d_fwd with the optional inputs of causal_conv1d_fn (same page
 * section 4.2: seq_idx, initial_states, return_final_states /
 * final_states_out).  Every pointer is a device pointer.
 *  - initial_states (batch, dim, width-1) io: the inputs before t = 0, oldest
 *    first (replacing the zero padding);
 *  - final_states (batch, dim, width-1) io, written: the last width-1 inputs
 *    of the row (with initial_states / zeros in front when seqlen < width-1),
 *    copied bit for bit -- the conv cache for continuing the sequence;
 *  - seq_idx (batch, seqlen) int32: packed sequences; a tap contributes only
 *    when its position carries the output's id, so each sequence restarts
 *    from zero.  Ids are expected to be contiguous per sequence.  seq_idx
 *    with initial_states or final_states returns SSM_ERR_UNSUPPORTED (the
 *    page: they cannot be used together).
 * width must be 4.  Same status codes as causal_conv1d_fwd. */
typedef struct causal_conv1d_args {
  int64_t batch, dim, seqlen;
  int32_t width, io_dtype, act;
  const void *x;                                /* (b,d,l) io, required */
  const float *weight;                          /* (d, width) fp32, required */
  const float *bias;                            /* (d) fp32 or NULL */
  const int32_t *seq_idx;                       /* (b,l) int32 or NULL */
  const void *initial_states;                   /* (b,d,width-1) io or NULL */
  void *out;                                    /* (b,d,l) io, required */
  void *final_states;                           /* (b,d,width-1) io or NULL */
} causal_conv1d_args_t;
int causal_conv1d_fwd_ex(const causal_conv1d_args_t *args, void *hip_stream);

/* Host-only argument check of causal_conv1d_fwd_ex (no HIP call). */
int causal_conv1d_ex_validate(const causal_conv1d_args_t *args);

/* Host-only argument check of causal_conv1d_fwd (no HIP call). */
int causal_conv1d_validate(const void *x, const float *weight, const void *out,
                           int64_t batch, int64_t dim, int64_t seqlen, int32_t width,
                           int32_t io_dtype, int32_t act);

/* ---------------------------------------------------------------------------
 * Single-step decode.
 * ------------------------------------------------------------------------- */

#define SSM_MAX_CONV_STATE 256  /* largest conv cache length causal_conv1d_update takes */

/* Arguments of ssm_state_update.  Every pointer is a device pointer. */
typedef struct ssm_state_update_args {
  int64_t batch, dim, dstate, ngroups;          /* ngroups: 1 unless grouped */
  int32_t io_dtype;                             /* SSM_F32 or SSM_BF16 */
  float *state;                                 /* (b,d,n) fp32: read, then overwritten */
  const void *x;                                /* (b,d) io, required */
  const void *dt;                               /* (b,d) io, required */
  const float *A;                               /* (d,n) fp32, required */
  const void *B;                                /* (b,g,n) io, required */
  const void *C;                                /* (b,g,n) io, required */
  const float *D;                               /* (d) fp32 or NULL */
  const float *dt_bias;                         /* (d) fp32 or NULL */
  const void *z;                                /* (b,d) io or NULL */
  int32_t dt_softplus;                          /* 0 or 1 */
  void *out;                                    /* (b,d) io, required */
} ssm_state_update_args_t;

/* selective_state_update: one decode step of the recurrence above against a
 * cached state (the PaddleNLP Kernel operator-library guide lists
 * selective_state_update among its mamba operators, section 4.4; it is not
 * printed there, and is read as one timestep of section 4.1's scan applied
 * to a cache).  For every (b, d), with dt' = softplus(dt + dt_bias) when
 * dt_softplus is set (otherwise dt + dt_bias) and g = d / (dim / ngroups):
 *
 *     state[b,d,s] <- exp(dt' * A[d,s]) * state[b,d,s] + dt' * B[b,g,s] * x[b,d]
 *     out[b,d]      = (sum_s C[b,g,s] * state[b,d,s] + D[d] * x[b,d]) * silu(z[b,d])
 *
 * (the contraction uses the updated state).  A Mamba-2 style state
 * (batch, nheads, headdim, dstate) is this call with dim = nheads * headdim
 * and every per-head tensor expanded over headdim.  The state is updated in
 * place and must not overlap any other argument; `out` must not alias an
 * input.  dstate <= SSM_MAX_DSTATE.  Same conventions and status codes as
 * ssm_scan_fwd; the update is a pure function of its inputs, so calls on one
 * stream compose into a sequence of decode steps. */
int ssm_state_update(const ssm_state_update_args_t *args, void *hip_stream);

/* Host-only argument check of ssm_state_update (no HIP call). */
int ssm_state_update_validate(const ssm_state_update_args_t *args);

/* causal_conv1d_update: the causal conv of causal_conv1d_fwd continued from a
 * cache of earlier inputs (same guide, section 4.2: single-step incremental
 * inference over a conv_state cache, with an optional ring buffer indexed by
 * cache_seqlens).  x: (batch, dim, seqlen) io, the new tokens; conv_state:
 * (batch, dim, state_len) io, state_len >= width - 1, read and updated in
 * place; weight: (dim, width) fp32; bias: (dim) fp32 or NULL; out: (batch,
 * dim, seqlen) io.  For every new token t,
 *
 *     out[b,d,t] = round_io(act(bias[d] + sum_k weight[d,k] * h[t - (width-1) + k]))
 *
 * where h is the input history: the inputs before the first new token come
 * from the cache, the rest are x.
 *  - cache_seqlens == NULL: the cache is ordered oldest first (its last
 *    width-1 entries precede x[.,.,0]); afterwards it holds the last state_len
 *    inputs of (cache, x).
 *  - cache_seqlens != NULL (device pointer, one int32 >= 0 per batch): the
 *    cache is a ring buffer; token t is written at slot
 *    (cache_seqlens[b] + t) % state_len and the inputs before it are the
 *    width-1 slots before that one, circularly.  Other slots are untouched
 *    and cache_seqlens is not advanced (the caller adds seqlen).
 * 2 <= width <= SSM_CONV_WIDTH, state_len <= SSM_MAX_CONV_STATE.  x, out and
 * conv_state must not overlap.  Asynchronous on hip_stream; returns a status
 * code. */
int causal_conv1d_update(const void *x, void *conv_state, const float *weight,
                         const float *bias, const int32_t *cache_seqlens, void *out,
                         int64_t batch, int64_t dim, int64_t seqlen, int64_t state_len,
                         int32_t width, int32_t io_dtype, int32_t act, void *hip_stream);

/* Host-only argument check of causal_conv1d_update (no HIP call). */
int causal_conv1d_update_validate(const void *x, const void *conv_state, const float *weight,
                                  const void *out, int64_t batch, int64_t dim, int64_t seqlen,
                                  int64_t state_len, int32_t width, int32_t io_dtype,
                                  int32_t act);

/* ---------------------------------------------------------------------------
 * Mamba-2 chunked scan (state-space duality form).
 * ------------------------------------------------------------------------- */

#define SSD_HEADDIM 64     /* the head width the kernel is built for */
#define SSD_CHUNK 64       /* tokens per chunk of the chunked evaluation */

/* Arguments of ssd_scan_fwd.  Every pointer is a device pointer; x, z, out,
 * B and C must be 16-byte aligned. */
typedef struct ssd_scan_args {
  int64_t batch, seqlen, nheads, headdim, dstate, ngroups;
  int32_t io_dtype;               /* SSM_BF16 */
  const void *x;                  /* (b,l,h,p) io, required */
  const void *dt;                 /* (b,l,h) io, required */
  const float *A;                 /* (h) fp32, required */
  const void *B;                  /* (b,l,g,n) io, required */
  const void *C;                  /* (b,l,g,n) io, required */
  const float *D;                 /* (h) or (h,p) fp32, or NULL */
  int32_t D_per_channel;          /* 1: D is (h,p) */
  const void *z;                  /* (b,l,h,p) io or NULL */
  const float *dt_bias;           /* (h) fp32 or NULL */
  int32_t dt_softplus;            /* 0 or 1 */
  const float *initial_states;    /* (b,h,p,n) fp32 or NULL (zero) */
  void *out;                      /* (b,l,h,p) io, required */
  float *final_states;            /* (b,h,p,n) fp32 or NULL */
  /* Step range (the operators' dt_limit): when dt_limit is 1 the step is
   * clamped, dt' = min(max(dt', dt_min), dt_max), after softplus; 0: no
   * clamp.  dt_min > dt_max returns SSM_ERR_SHAPE. */
  int32_t dt_limit;
  float dt_min, dt_max;
  /* Packed sequences (the operators' seq_idx): (b,l) int32 sequence ids, or
   * NULL.  Ids must not decrease along l (each sequence is one contiguous
   * run); where the id changes the state restarts from zero, so no token
   * sees a token of another sequence.  initial_states is the state before
   * the first sequence of each row, final_states the state after the last.
   * Ids that decrease give unspecified results (never a fault). */
  const int32_t *seq_idx;
  /* Scratch for the sequence split (see ssd_scan_workspace_size): caller-
   * allocated device memory; the library allocates nothing and returns
   * SSM_ERR_WORKSPACE when the plan needs more than workspace_bytes.  Not
   * read before written; reusable once the call's work has finished. */
  void *workspace;
  size_t workspace_bytes;
  /* Sequence split: 0 lets the library choose (its segments may differ in
   * length); k >= 1 asks for k segments of ceil(chunks / k) whole chunks,
   * the last one taking the rest (possibly fewer segments).  Negative values
   * return SSM_ERR_SHAPE.  The split changes the results only by rounding
   * order. */
  int32_t seq_segments;
} ssd_scan_args_t;

/* ssd_scan_fwd: the Mamba-2 chunked scan (the guide's section 4.4 lists
 * mamba_chunk_scan_combined, chunk_state and state_passing among its mamba
 * operators without printing them; they are read as the selective-scan
 * recurrence with a scalar decay per head, evaluated chunk by chunk).  For
 * every (b, h), head h in group g = h / (nheads / ngroups), and token t:
 *
 *     dt'          = softplus(dt[b,t,h] + dt_bias[h])   (or without softplus;
 *                    then clamped to [dt_min, dt_max] with dt_limit)
 *     H[p][n]     <- 0 first where seq_idx[b,t] != seq_idx[b,t-1]
 *     H[p][n]     <- exp(dt' * A[h]) * H[p][n] + dt' * B[b,t,g,n] * x[b,t,h,p]
 *     out[b,t,h,p] = (sum_n C[b,t,g,n] * H[p][n] + D * x[b,t,h,p]) * silu(z[b,t,h,p])
 *
 * with H starting at initial_states and its last value stored to
 * final_states.  The kernel evaluates each chunk of SSD_CHUNK tokens in the
 * quadratic (dual) form on the matrix cores -- products of bf16 operands
 * accumulated in fp32 -- and carries the fp32 state from chunk to chunk.
 * When batch * nheads alone leaves the GPU short of workgroups, the chunks
 * are cut into segments: a first launch finds each segment's end state
 * from zero and its total decay (chunk_state), the second starts every
 * segment from the state carried over the ones before it (state_passing)
 * and computes the outputs (chunk_scan).
 * Supported: io_dtype SSM_BF16, headdim SSD_HEADDIM, dstate 32, 64 or 128;
 * other values return SSM_ERR_UNSUPPORTED.  Same conventions and status
 * codes as ssm_scan_fwd. */
int ssd_scan_fwd(const ssd_scan_args_t *args, void *hip_stream);

/* Host-only argument check of ssd_scan_fwd (no HIP call). */
int ssd_scan_validate(const ssd_scan_args_t *args);

/* Scratch bytes ssd_scan_fwd needs for these arguments (0 without a
 * sequence split).  Host-only apart from cached queries of the device's
 * compute-unit count and the kernels' occupancy. */
int ssd_scan_workspace_size(const ssd_scan_args_t *args, size_t *bytes);

/* The three parts of mamba_chunk_scan_combined as section 4.4 of the guide
 * names them (chunk_state, state_passing, the chunk scan), over chunks of
 * chunk_size tokens (a positive multiple of SSD_CHUNK; the last chunk may be
 * shorter); nchunks = ceil(seqlen / chunk_size).  Per (b, h) the scan of
 * chunk c maps the state entering it affinely, H_end = P_c H_start + E_c,
 * and the three calls composed give ssd_scan_fwd's out and final_states:
 *
 *   ssd_chunk_state:   E_c, the chunk's end state from a zero state, into
 *                      states (nchunks,b,h,p,n) fp32, and P_c into decays
 *                      (nchunks,b,h) fp32: exp(A[h] * the chunk's summed
 *                      steps), or 0 where seq_idx changes at one of the
 *                      chunk's tokens (t > 0), the first included.  Reads
 *                      x, dt, A, B, dt_bias, dt_softplus, dt_limit and
 *                      seq_idx of args (C, D, z, out, the states, workspace
 *                      and seq_segments are ignored and may be NULL).
 *   ssd_state_passing: carried[c] = S_c with S_0 = initial_states (zero
 *                      when NULL) and S_{c+1} = decays[c] S_c + states[c],
 *                      each step one fp32 fma; final_states (b,h,p,n), if
 *                      not NULL, gets S_nchunks.  Plain device arrays of
 *                      the layouts above; carried (nchunks,b,h,p,n) fp32.
 *   ssd_chunk_scan:    out of every chunk from the state carried[c] (the
 *                      whole of args but initial_states, which carried[0]
 *                      replaces, and workspace / seq_segments, which are
 *                      ignored), and the state after the last chunk into
 *                      final_states when given.
 *
 * Same supported sizes, alignment, conventions and status codes as
 * ssd_scan_fwd; a chunk_size that is not a positive multiple of SSD_CHUNK
 * returns SSM_ERR_UNSUPPORTED.  None of them needs scratch.  The *_validate
 * calls are the host-only checks (no HIP call). */
int ssd_chunk_state(const ssd_scan_args_t *args, int64_t chunk_size, float *states, float *decays,
                    void *hip_stream);
int ssd_chunk_state_validate(const ssd_scan_args_t *args, int64_t chunk_size, const float *states,
                             const float *decays);
int ssd_state_passing(int64_t nchunks, int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                      const float *states, const float *decays, const float *initial_states,
                      float *carried, float *final_states, void *hip_stream);
int ssd_state_passing_validate(int64_t nchunks, int64_t batch, int64_t nheads, int64_t headdim,
                               int64_t dstate, const float *states, const float *decays,
                               const float *carried);
int ssd_chunk_scan(const ssd_scan_args_t *args, int64_t chunk_size, const float *carried, void *hip_stream);
int ssd_chunk_scan_validate(const ssd_scan_args_t *args, int64_t chunk_size, const float *carried);

/* Static text for a status code. */
const char *ssm_status_str(int status);

/* The hipError_t of the last SSM_ERR_HIP returned on this thread (0 if none). */
int ssm_last_hip_error(void);

/* SSM_ABI_VERSION of the loaded library. */
int ssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSMSCAN_H */
