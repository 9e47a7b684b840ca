/*
 * ssm_scan.h -- C ABI of libssmscan.so, the selective state-space scan
 * (Mamba's S6 layer core) for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every batch row b, channel d and state n the library
 * runs one diagonal single-input single-output state-space model:
 *
 *   Abar_t[n] = exp(Delta[b,t,d] * A[d,n])
 *   Bbar_t[n] = Delta[b,t,d] * B[b,t,n]                       (SSM_DISC_DELTA_B)
 *             = (exp(Delta[b,t,d] A[d,n]) - 1) / A[d,n] * B[b,t,n]   (SSM_DISC_ZOH)
 *   h_t[n]    = Abar_t[n] * h_{t-1}[n] + Bbar_t[n] * u[b,t,d]
 *   y[b,t,d]  = sum_n C[b,t,n] * h_t[n] + Dskip[d] * u[b,t,d]
 *
 * with h_{-1} = h0 (zero when h0 is NULL) and u the scan input: x itself, or
 * the causal depthwise conv1d + SiLU of x when conv_w is given,
 *
 *   u[b,t,d] = silu(conv_b[d] + sum_{k<K} conv_w[d,k] * x[b, t-K+1+k, d]),
 *   x[b, t<0, d] = conv_state_in[b, d, K-1+t] (0 when conv_state_in is NULL),
 *   silu(z) = z / (1 + exp(-z)).
 *
 * Optional fused steps around the scan:
 *   - step size from its pre-activation: Delta = delta + delta_bias[d], and
 *     with delta_softplus Delta = softplus(delta + delta_bias[d]),
 *     softplus(v) = log(1 + exp(v));
 *   - output gate: y[b,t,d] is multiplied by silu(z[b,t,d]);
 *   - conv window across calls: conv_state_out[b, d, j] = x[b, L-K+1+j, d]
 *     (the last K-1 inputs, oldest first, reaching into conv_state_in when
 *     L < K-1), so a sequence scanned in pieces, or a prefill followed by
 *     ssm_step calls, sees the same window as one call.
 *
 * Passages defining each step (web pages on Mamba; section names as printed):
 *   - continuous SSM, ZOH discretization Abar = exp(Delta A),
 *     Bbar = (Delta A)^-1 (exp(Delta A) - I) Delta B, and the discrete
 *     recurrence h_k = Abar h_{k-1} + Bbar x_k, y_k = C h_k + D x_k:
 *     gsyq.cn "Mamba 状态空间模型深度解析", section "连续到离散的转换";
 *   - the simplified Bbar = Delta * B and the scan h = associative_scan(
 *     A_bar, B_bar * x), y = C * h: same page, section "硬件优化并行扫描算法";
 *   - A kept continuous and discretized on the fly; one independent SSM per
 *     channel with A (D, N), B and C (batch, L, N), Delta (batch, L, D); C is
 *     a 1 x N row, so the readout contracts over n: VMamba reading note,
 *     sections "离散化SSM", "S4中三个矩阵的维度表示、维度变化" and
 *     "mamba：从S4到S6的算法变化流程";
 *   - the causal depthwise Conv1d (padding d_conv - 1, groups = d_model) before
 *     the SSM and the skip D * x_conv on the conv output: gsyq.cn section
 *     "选择性的实现细节" (SelectiveSSM);
 *   - the single-token recurrent step with a cached state (constant cost per
 *     generated token): 53ai.com explainer, section "一、Motivation", and the
 *     datacamp tutorial's complexity table;
 *   - Delta = Softplus(Linear(x)), the bias of that projection being
 *     delta_bias: gsyq.cn section "选择性的数学解析"; VMamba note section
 *     "mamba：从S4到S6的算法变化流程" (tau_Delta = softplus);
 *   - the gated block around the SSM (H3 block merged with a gated MLP):
 *     VMamba note section "简化的SSM架构".  The page's figure with the gate
 *     formula is lost; y * silu(z), applied after the skip term, is the
 *     reading taken.
 *
 * Conventions shared by every entry point.
 *   Layout     all arrays are dense, row-major, last dimension fastest:
 *              x, Delta, y (batch, L, D); B, C (batch, L, N); A (D, N);
 *              Dskip, conv_b, delta_bias (D); conv_w (D, K); h0, h_last
 *              (batch, D, N); z like x; conv_state_in / conv_state_out
 *              (batch, D, K-1) fp32, oldest input first.
 *              Base pointers must be aligned to their element size; B and C
 *              rows are read with scalar loads, so B and C base pointers must
 *              be 4-byte aligned and are best 64-byte aligned.
 *   Memory     every pointer is a DEVICE pointer owned by the caller.  The
 *              library allocates nothing, keeps no pointer after the call and
 *              holds no global mutable state apart from the scratch array of
 *              ssm_scan_fwd_noalloc and its per-device address table; every
 *              entry point except that one is reentrant and thread-safe.
 *   Streams    hip_stream is a hipStream_t (NULL = the default stream).  Work
 *              is enqueued asynchronously; the call never synchronizes.  A
 *              call enqueues kernel launches only (plus the optional timing
 *              events), with no memset or copy, so it may be recorded by
 *              stream capture into a HIP graph and replayed; a replay reads
 *              the buffers whose addresses were passed when it was captured.
 *   Errors     all argument checks run on the host before anything is
 *              enqueued; on any error the outputs are untouched and the
 *              status says why (ssm_last_error_message() has the detail).  A
 *              failed launch returns SSM_ERR_HIP; faults inside kernels
 *              surface at the caller's next synchronization.
 *   Dtypes     x, Delta, B, C, z share in_dtype (fp32 or bf16); y has
 *              out_dtype; A, Dskip, delta_bias, conv weights, conv states and
 *              h are fp32; arithmetic and the state are fp32; bf16 outputs are
 *              rounded to nearest even.
 *   Empty      seqlen == 0 or batch * dim == 0 is valid.  With seqlen == 0 and
 *              batch * dim > 0, h_last (if given) receives h0 (zeros if h0 is
 *              NULL), conv_state_out (if given) receives conv_state_in (zeros
 *              if NULL), and nothing else is touched.
 */
#ifndef SSM_SCAN_H_
#define SSM_SCAN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 3

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = 1,        /* a required pointer (or the args struct) is NULL */
  SSM_ERR_SHAPE = 2,       /* negative sizes, or byte counts overflow int64 */
  SSM_ERR_DTYPE = 3,       /* unknown dtype or discretization enum value */
  SSM_ERR_UNSUPPORTED = 4, /* dstate not in {1,2,4,8,16}, conv_k not in 1..4,
                              misaligned pointer, negative chunk_len, reserved != 0,
                              delta_softplus not 0/1, conv state without conv_w,
                              h_saved with a split scan whose chunk_len is not a
                              multiple of 4 */
  SSM_ERR_ALIAS = 5,       /* an output overlaps an input or another output */
  SSM_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required */
  SSM_ERR_HIP = 7          /* the HIP runtime rejected a launch */
} ssm_status_t;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype_t;

typedef enum { SSM_DISC_DELTA_B = 0, SSM_DISC_ZOH = 1 } ssm_disc_t;

typedef struct {
  int64_t batch, seqlen, dim, dstate; /* Bt, L, D, N */
  int32_t in_dtype;                   /* ssm_dtype_t of x, delta, Bm, Cm */
  int32_t out_dtype;                  /* ssm_dtype_t of y */
  int32_t disc;                       /* ssm_disc_t */
  int32_t conv_k;                     /* taps of the conv prologue (1..4); ignored if conv_w is NULL */
  const void* x;                      /* (Bt, L, D) */
  const void* delta;                  /* (Bt, L, D), the step size, already positive */
  const float* A;                     /* (D, N), continuous-time diagonal */
  const void* Bm;                     /* (Bt, L, N) */
  const void* Cm;                     /* (Bt, L, N) */
  const float* Dskip;                 /* (D) or NULL = no skip term */
  const float* h0;                    /* (Bt, D, N) or NULL = zero initial state */
  float* h_last;                      /* (Bt, D, N) or NULL: state after the last token */
  void* y;                            /* (Bt, L, D) output */
  const float* conv_w;                /* (D, K) or NULL = no conv prologue */
  const float* conv_b;                /* (D) or NULL = zero bias */
  void* workspace;                    /* device scratch of >= ssm_scan_workspace_size() bytes */
  size_t workspace_bytes;
  int32_t chunk_len;                  /* time steps per chunk; 0 = library's choice */
  int32_t reserved;                   /* must be 0 */
  void* ev_main_start;                /* optional hipEvent_t recorded on hip_stream right */
  void* ev_main_stop;                 /* before / after the output-pass kernel; NULL = none */
  /* since ABI 2 */
  const float* delta_bias;            /* (D) or NULL = 0, added to delta */
  int32_t delta_softplus;             /* 1: Delta = softplus(delta + delta_bias); 0: no softplus */
  int32_t reserved2;                  /* must be 0 */
  const void* z;                      /* (Bt, L, D) gate or NULL = no gate: y *= silu(z) */
  const float* conv_state_in;         /* (Bt, D, K-1) inputs before token 0, or NULL = zeros;
                                         requires conv_w */
  float* conv_state_out;              /* (Bt, D, K-1) receives the last K-1 inputs, or NULL;
                                         requires conv_w; must not overlap any other buffer */
  /* since ABI 3 */
  float* h_saved;                     /* (Bt, S, D, N) fp32 or NULL, S = ceil(L / 16) - 1:
                                         receives the state entering steps 16, 32, ..., 16 S
                                         (h_saved[b][k-1] = h before step 16 k), for
                                         ssm_scan_bwd; must not overlap any other buffer.
                                         When the scan is split into chunks, their length
                                         must be a multiple of 4 (the planned length is) */
} ssm_scan_args_t;

typedef struct {
  int64_t batch, dim, dstate;         /* Bt, D, N */
  int32_t in_dtype;                   /* ssm_dtype_t of x, delta, Bm, Cm */
  int32_t out_dtype;                  /* ssm_dtype_t of y */
  int32_t disc;                       /* ssm_disc_t */
  int32_t reserved;                   /* must be 0 */
  const void* x;                      /* (Bt, D) the new token's scan input */
  const void* delta;                  /* (Bt, D) */
  const float* A;                     /* (D, N) */
  const void* Bm;                     /* (Bt, N) */
  const void* Cm;                     /* (Bt, N) */
  const float* Dskip;                 /* (D) or NULL */
  float* h;                           /* (Bt, D, N) cached state, updated in place;
                                         aligned to 4 * min(N, 4) bytes */
  void* y;                            /* (Bt, D) output, read from the updated state */
  /* since ABI 2 */
  const float* delta_bias;            /* (D) or NULL = 0, added to delta */
  int32_t delta_softplus;             /* 1: Delta = softplus(delta + delta_bias) */
  int32_t conv_k;                     /* taps of the conv (1..4); ignored if conv_w is NULL */
  const void* z;                      /* (Bt, D) gate or NULL: y *= silu(z) */
  const float* conv_w;                /* (D, K) or NULL = no conv: u = x */
  const float* conv_b;                /* (D) or NULL = zero bias */
  float* conv_state;                  /* (Bt, D, K-1) conv window, updated in place (shifted to
                                         end with x); required when conv_w is given and K > 1 */
} ssm_step_args_t;

/* Backward selective scan: gradients of
 *   loss = sum(dy * y) + sum(dh_last * h_last)
 * for ssm_scan_fwd without fused steps (no conv prologue, Delta as given, no
 * gate).  The derivative of the recurrence defined above (the pages name
 * training as the purpose of the parallel scan -- explainer, section "3.6
 * Empirical Evaluation"; VMamba note, section "硬件感知的设计" -- and print
 * no gradient formula; the chain rule of the definition is the reading):
 *   g_t = C_t dy_t + Abar_{t+1} g_{t+1} (g_{L-1} also receives dh_last),
 *   dx_t = sum_n g_t f_t B_t + Dskip dy_t, dDelta_t, dA, dB, dC, dD, dh0.
 * All gradients are fp32 and overwritten (not accumulated).  Inputs are as
 * in ssm_scan_args_t; dy has in_dtype.  The adjoint is chunked like the
 * forward scan and the forward states are recomputed between states kept
 * every 16 steps, so nothing of size batch x L x D x N is stored.  The
 * states every 16 steps are either computed here (a forward summary and
 * carry pass) or taken from the forward scan of the same inputs (h_saved of
 * ssm_scan_args_t), which skips that pass. */
typedef struct {
  int64_t batch, seqlen, dim, dstate; /* Bt, L, D, N */
  int32_t in_dtype;                   /* ssm_dtype_t of x, delta, Bm, Cm, dy */
  int32_t disc;                       /* ssm_disc_t */
  int32_t super_chunk;                /* steps per adjoint chunk (multiple of 16); 0 = plan */
  int32_t reserved;                   /* must be 0 */
  const void* x;                      /* (Bt, L, D) */
  const void* delta;                  /* (Bt, L, D) */
  const float* A;                     /* (D, N) */
  const void* Bm;                     /* (Bt, L, N) */
  const void* Cm;                     /* (Bt, L, N) */
  const float* Dskip;                 /* (D) or NULL */
  const float* h0;                    /* (Bt, D, N) or NULL */
  const void* dy;                     /* (Bt, L, D) gradient of y */
  const float* dh_last;               /* (Bt, D, N) gradient of h_last, or NULL */
  float* dx;                          /* (Bt, L, D) */
  float* ddelta;                      /* (Bt, L, D) */
  float* dA;                          /* (D, N) */
  float* dB;                          /* (Bt, L, N) */
  float* dC;                          /* (Bt, L, N) */
  float* dD;                          /* (D) or NULL */
  float* dh0;                         /* (Bt, D, N) or NULL */
  void* workspace;                    /* >= ssm_scan_bwd_workspace_size() bytes */
  size_t workspace_bytes;
  void* ev_main_start;                /* optional hipEvent_t recorded on hip_stream right */
  void* ev_main_stop;                 /* before / after the main backward kernel; NULL = none */
  /* since ABI 3 */
  const float* h_saved;               /* (Bt, ceil(L / 16) - 1, D, N) or NULL: the states
                                         ssm_scan_fwd wrote to its h_saved for the same x,
                                         delta, A, Bm, h0 (and disc); NULL = computed here */
} ssm_scan_bwd_args_t;

/* Bytes of device scratch the allocation-free forward entry point holds per
 * GPU (see ssm_scan_fwd_noalloc). */
#define SSM_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Returns SSM_ABI_VERSION. */
int ssm_abi_version(void);

/* Bytes of device workspace ssm_scan_fwd needs for these arguments (0 when the
 * plan scans each sequence in one piece).  Reads only the sizes, chunk_len and
 * dtypes; pure host function, no HIP call.  Returns 0 for invalid sizes. */
size_t ssm_scan_workspace_size(const ssm_scan_args_t* args);

/* Time steps per chunk the plan uses for these arguments (equal to seqlen
 * when the scan is not split).  Pure host function; 0 for invalid sizes.
 * With chunk_len = 0, sequences of at most 32 steps are not split, and short
 * sequences of few channels (seqlen <= 512 and batch * dim * ceil(seqlen /
 * 64) <= min(4096, 64 * seqlen)) run as one
 * pass with the time steps across a wave's lanes, each block of 64 steps
 * solved by a parallel associative scan over the lanes (53ai.com explainer,
 * section 3.3); that plan reports seqlen and needs no workspace. */
int64_t ssm_scan_plan_chunk_len(const ssm_scan_args_t* args);

/* 1 when the plan for these arguments is that one-pass lane scan (one
 * kernel, k_scan_wave), 0 when it is the chunked passes (chunk summaries,
 * carry combine and output pass; a single chunk runs the output pass alone)
 * or the sizes are invalid.  Pure host function, no HIP call. */
int32_t ssm_scan_plan_lane_scan(const ssm_scan_args_t* args);

/* Selective-scan forward: y and (optionally) h_last from the inputs above.
 * The time axis may be split into chunks scanned in parallel; their carries
 * are combined with the associative operator
 *   (a, b) o (a', b') = (a a', a' b + b')
 * which is exact up to floating-point rounding order. */
ssm_status_t ssm_scan_fwd(const ssm_scan_args_t* args, void* hip_stream);

/* ssm_scan_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops, and harnesses that forbid hipMalloc.
 * Same arguments and results as ssm_scan_fwd, except that workspace and
 * workspace_bytes are ignored: the chunk summaries, carries and group
 * carries live in a device array of SSM_NOALLOC_SCRATCH_BYTES that the
 * library keeps on every GPU it runs on, until the process ends.  The call
 * allocates nothing.
 *   - Plan: the library's plan when its summaries fit the array; otherwise
 *     the same plan with chunks lengthened until they do (results then
 *     differ from ssm_scan_fwd's by rounding order only).  A chunk_len the
 *     caller forces is kept, and the call fails with SSM_ERR_WORKSPACE if
 *     its summaries do not fit.  ssm_scan_plan_chunk_len reports the
 *     ordinary plan, not this one.
 *   - The array's device address is looked up (hipGetSymbolAddress) on the
 *     first call on each device that needs it, with that device current;
 *     make that first call outside stream capture.  hip_stream must belong
 *     to the current device (SSM_ERR_UNSUPPORTED otherwise).
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (concurrent streams, or threads) race and corrupt each
 *     other's results.  Serialize them, e.g. on one stream.  Nothing in the
 *     array needs clearing between calls; it keeps the last call's contents.
 * Errors as for ssm_scan_fwd. */
ssm_status_t ssm_scan_fwd_noalloc(const ssm_scan_args_t* args, void* hip_stream);

/* One recurrent decode step per sequence: u = x (or the conv over the
 * window conv_state followed by x, then SiLU), h <- Abar h + Bbar u, then
 * y = (C . h + Dskip * u) (* silu(z)), with h and conv_state updated in
 * place.  Same arithmetic as ssm_scan_fwd with seqlen = 1, h0 = h_last = h
 * and conv_state_in = conv_state_out = conv_state.  y must not overlap h,
 * conv_state or any input. */
ssm_status_t ssm_step(const ssm_step_args_t* args, void* hip_stream);

/* Bytes of device workspace ssm_scan_bwd needs (never 0 for a non-empty
 * problem; smaller when h_saved is given).  Pure host function; 0 for
 * invalid sizes. */
size_t ssm_scan_bwd_workspace_size(const ssm_scan_bwd_args_t* args);

/* Backward selective scan (see ssm_scan_bwd_args_t).  Asynchronous on
 * hip_stream; outputs must not overlap each other, the inputs or the
 * workspace.  Errors as for ssm_scan_fwd. */
ssm_status_t ssm_scan_bwd(const ssm_scan_bwd_args_t* args, void* hip_stream);

/* Static description of a status code. */
const char* ssm_status_string(ssm_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* ssm_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H_ */
