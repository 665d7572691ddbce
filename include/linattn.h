/*
 * linattn.h -- C ABI of liblinattn.so: causal linear attention with an
 * elu+1 feature map, optional per-head decay, eps-stabilised normaliser,
 * and the gated delta rule, as a chunked prefill over whole sequences and as
 * a single-token decode step against a persistent state.  gfx950 (MI355X).
 *
 * Sources (web pages, cited by title and section):
 *   "What Is Linear Attention?" (xutianle.me)                       [WILA]
 *   "Efficient attention variants" (bailixisu.com)                   [EAV]
 *   "LLM inference optimisation (3): Linear Attention" (wangyu.me)   [LIO3]
 *   "Transformers Are RNNs" (myhz0606.com)                           [TAR]
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers to contiguous row-major memory
 *     owned by the caller.  The library never allocates, frees or keeps a
 *     pointer after the call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and runs asynchronously; the library never synchronises the
 *     host.  The caller must keep every buffer alive until the stream has
 *     passed the enqueued work.
 *   - Arguments are validated before anything is enqueued: a call that
 *     returns LA_EINVAL, LA_EUNSUPPORTED or LA_EWORKSPACE has enqueued
 *     nothing.  LA_EHIP means a HIP launch failed; work enqueued before the
 *     failure may still run.  The library never aborts and never throws
 *     across this interface.
 *   - B, H and N may be 0 (nothing to do); d and dv are 1..128.
 *   - Thread-safe: the only shared state is a cached per-device CU count
 *     and the (mutex-guarded) kernel timing log below.
 *   - Results are deterministic for a given device, shape and build: no
 *     atomics take part in any sum.
 *   - Numerics: inputs fp32 or bf16; feature maps, decays, normaliser,
 *     state and all accumulation in fp32.  With bf16 inputs the matrix
 *     products take bf16 operands (the state read uses a bf16 copy of the
 *     fp32 state; the fp32 state itself is never rounded).
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_MAX_DIM 128 /* largest d and dv */

typedef enum {
  LA_OK = 0,
  LA_EINVAL = 1,       /* a NULL pointer where one is required, a negative
                          size, d or dv outside 1..128, eps < 0 or not finite,
                          or an argument the rule does not take */
  LA_EUNSUPPORTED = 2, /* valid request the library does not implement */
  LA_EHIP = 3,         /* a HIP call or kernel launch failed */
  LA_EWORKSPACE = 4,   /* workspace NULL or smaller than
                          la_prefill_workspace_size() */
  LA_ESCRATCH = 5      /* la_prefill_noalloc: the call needs more workspace
                          than LA_NOALLOC_SCRATCH_BYTES */
} la_status;

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype; /* dtype of q, k, v, o */

/* The feature map phi applied to q and k ([EAV] section 4, [LIO3] 'what is
 * phi'): ELU1 is elu(x)+1 with alpha 1, i.e. x+1 for x > 0 and e^x
 * otherwise; IDENTITY means q and k already are the (non-negative) features,
 * as in the hand-worked example of [EAV] section 5.1. */
typedef enum { LA_FMAP_IDENTITY = 0, LA_FMAP_ELU1 = 1 } la_fmap;

/* LA_RULE_LINEAR ([WILA] sections 4 and 5.1; [EAV] section 5; [TAR] eps):
 *     S_t = gamma_h S_{t-1} + phi(k_t) v_t^T,  z_t = gamma_h z_{t-1} + phi(k_t)
 *     o_t = S_t^T phi(q_t) / (phi(q_t) . z_t + eps)
 *   The state is read after the token is written (the token sees itself).
 *   Instead of gamma, a per-key-channel decay alpha_t (GLA, [EAV] section
 *   7.2) scales each state row and z entry by its own factor:
 *     S_t = diag(alpha_t) S_{t-1} + phi(k_t) v_t^T,  z_t = alpha_t . z_{t-1} + phi(k_t)
 * LA_RULE_DELTA ([WILA] sections 5.2 and 5.3):
 *     S_t = S_{t-1} + g_t k_t (v_t - S_{t-1}^T k_t)^T,   o_t = S_t^T q_t
 *   raw q and k (fmap must be IDENTITY), no normaliser, no z.  With the
 *   optional scalar decay alpha_t (Gated DeltaNet, [EAV] section 7.4; the
 *   error is taken on the decayed state):
 *     S_t = alpha_t S_{t-1} + g_t k_t (v_t - alpha_t S_{t-1}^T k_t)^T
 *
 * Short causal convolution (either rule; [WILA] section 5.4: a short
 * convolution over the most recent tokens in front of the state, with a
 * conv cache of those tokens kept beside the state for decoding): with
 * filters W [H, w, 2d+dv] (fp32, channels [q | k | v]) each raw q, k and v
 * channel is replaced, before the feature map (LINEAR) or the delta rule, by
 *     x'_t[c] = sum_{j=0..w-1} W[h, j, c] * x_{t-(w-1)+j}[c]
 * (tap w-1 on the current token; depthwise, no bias, no activation, and for
 * DELTA no normalisation of the convolved keys: the pages give none).  The
 * conv cache [B, H, w-1, 2d+dv] (dtype of q, rows oldest first) holds the
 * raw tokens before the current one: [q | k | v] of each token.  The DELTA
 * prefill convolves into copies of q, k, v in the workspace (rounded to
 * the dtype of q) and runs the rule on them. */
typedef enum { LA_RULE_LINEAR = 0, LA_RULE_DELTA = 1 } la_rule;

/* One call processes B*H independent sequences of N tokens. */
typedef struct la_prefill_args {
  int32_t B, H, N;   /* batch, heads, tokens per sequence (each >= 0) */
  int32_t d, dv;     /* key/query feature dim r = d; value dim (1..128) */
  int32_t dtype;     /* la_dtype of q, k, v and o */
  int32_t rule;      /* la_rule */
  int32_t fmap;      /* la_fmap (DELTA: IDENTITY only) */
  const void *q;     /* [B,H,N,d]  */
  const void *k;     /* [B,H,N,d]  */
  const void *v;     /* [B,H,N,dv] */
  const float *gamma;/* LINEAR: [H] decay per head, each in (0, 1]; NULL = 1.
                        DELTA: must be NULL.  Values are the caller's
                        contract (not read on the host).  Every decay factor
                        the kernels apply is a power gamma^m with m >= 0;
                        below gamma = 2^-40 the earlier tokens' weights are
                        taken as powers of 2^-40 (under 2^-40 of the
                        token's own, below fp32 resolution). */
  const float *g;    /* DELTA: [B,H,N] write gate per token (required).
                        LINEAR: must be NULL. */
  const float *alpha;/* State decay per token, or NULL (= 1, no decay).
                        DELTA: [B,H,N], each in (0, 1].
                        LINEAR: [B,H,N,d], one factor per key channel, each
                        in (0, 1]; not together with gamma.  Factors below
                        2^-15 are taken as 2^-15 (an earlier token then
                        weighs under 3.1e-5 of the current one).
                        Values are the caller's contract (not read on the
                        host); values outside the range make the chunk's
                        decay products inaccurate or undefined. */
  const float *conv_weight; /* [H, w, 2d+dv] short-convolution filters
                        (see above), or NULL (no convolution; then
                        conv_width is 0 and conv_in, conv_out are NULL). */
  int32_t conv_width;/* w, 1..4 with conv_weight */
  const void *conv_in;/* [B,H,w-1,2d+dv] conv cache before the sequence,
                        dtype as q; NULL = zeros */
  void *conv_out;    /* [B,H,w-1,2d+dv] the last w-1 raw tokens after the
                        sequence (from conv_in where N < w-1); NULL = not
                        written.  May alias conv_in exactly; no other
                        overlap. */
  float eps;         /* LINEAR: added to the denominator, >= 0. DELTA: ignored */
  const float *S_in; /* [B,H,d,dv] initial state; NULL = zeros */
  const float *z_in; /* LINEAR: [B,H,d] initial normaliser; NULL = zeros.
                        DELTA: must be NULL. */
  float *S_out;      /* [B,H,d,dv] state after the last token; NULL = not
                        written.  May alias S_in exactly (in-place update). */
  float *z_out;      /* LINEAR: [B,H,d]; NULL = not written; may alias z_in.
                        DELTA: must be NULL. */
  void *o;           /* [B,H,N,dv] output, dtype as q (required if N > 0) */
  float *den_out;    /* LINEAR: [B,H,N] each token's denominator
                        phi(q_t).z_t + eps (what la_backward needs), or NULL
                        (not written); with gamma or alpha alike.
                        With conv_weight the convolution then runs as a pass
                        of its own, into convolved copies of q, k, v at the
                        start of the workspace (la_backward's fwd_workspace
                        reads them).  DELTA: must be NULL. */
  void *workspace;   /* device scratch of workspace_bytes, caller-owned;
                        may be NULL when la_prefill_workspace_size() is 0.
                        DELTA, and LINEAR with den_out and conv_weight
                        together: 16-byte aligned (else LA_EINVAL).  Other
                        LINEAR calls: 4-byte aligned; 16-byte alignment with
                        d % 4 == 0 lets the kernels move it with vector
                        accesses. */
  size_t workspace_bytes;
} la_prefill_args;

/* Bytes of device workspace la_prefill needs for these arguments on the
 * current device (0 when none).  Reads only the sizes, dtype, rule,
 * conv_width and whether conv_weight, alpha and den_out are set.
 * Returns (size_t)-1 when the sizes are invalid. */
size_t la_prefill_workspace_size(const la_prefill_args *args);

/* Chunked prefill: computes o for every token and, when S_out/z_out are
 * given, the final state.  Equivalent (up to fp rounding order) to running
 * the per-token recurrence of `rule` from (S_in, z_in). */
int la_prefill(const la_prefill_args *args, void *stream);

/* la_prefill for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same computation and kernels as la_prefill (bit-identical results),
 * with the workspace taken from a static device array of
 * LA_NOALLOC_SCRATCH_BYTES that each GPU holds until the process ends (its
 * device address is looked up once per device, on the first call there,
 * with that device current).  The call allocates and frees nothing.
 * args->workspace must be NULL and workspace_bytes 0 (LA_EINVAL otherwise).
 * A call whose la_prefill_workspace_size() exceeds the array returns
 * LA_ESCRATCH and enqueues nothing; LA_EHIP if the array's address cannot be
 * obtained.  Every call on one GPU uses the same array: calls that overlap
 * on a GPU (other streams or threads) race, so the caller serialises them;
 * nothing needs clearing between calls (every element a call reads it has
 * written first). */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20) /* 128 MiB */
int la_prefill_noalloc(const la_prefill_args *args, void *stream);

/* Backward of a LINEAR-rule prefill (training).  The pages motivate
 * parallel training ([WILA] section 8; [EAV] sections 8 and 10) but give no
 * gradient formulas; these are the reverse-mode derivatives of the
 * recurrence above:
 *   dn_t = [g_t / den_t | -(g_t . o_t) / den_t]   (g_t = dL/do_t)
 *   adjoint state (backward in time), with the final-state gradient:
 *     Sh_t = phi(q_t) dn_t^T + gamma Sh_(t+1)   ([S | z] stacked, as dn)
 *   dphi(q_t) = [S_t | z_t] dn_t,  dphi(k_t) = Sh_t [v_t | 1],
 *   dv_t = (Sh_t^T phi(k_t)) without its last entry,
 *   dq = dphi(q) phi'(q), dk = dphi(k) phi'(k); dL/d(initial state) = gamma Sh_0.
 * With a per-key-channel decay alpha (GLA) in place of gamma the adjoint is
 * carried through diag(alpha_t), and
 *   dalpha_t[f] = sum_c Sh_t[f, c] S_(t-1)[f, c] + zh_t[f] z_(t-1)[f]
 * (S_(-1) the initial state), computed as (C0 + sum_(s>=t) (phi(q_s)
 * dphi(q_s) - phi(k_s) dphi(k_s))[f]) / alpha_t[f] with C0 = sum_c dS_out
 * S_N + dz_out z_N (the same sum, telescoped along the recurrence); alpha
 * below 2^-15, which the forward takes as 2^-15, gets dalpha 0.
 * Inputs are the forward's q, k, v, gamma or alpha, initial state, its
 * output o and its denominators den (la_prefill's den_out); with the
 * forward's convolution (conv_weight below) the gradients are taken
 * through it too.  Any d, dv up to 128 for both
 * dtypes; fp32 with d and dv both above 64 runs over the value columns
 * [0, 64) and [64, dv) in turn (the fp32 tiles of the whole width do not
 * fit the LDS; the gradients are linear in the value columns, so dq, dk and
 * dL/dz_in are sums over the halves) and then needs a workspace at any N;
 * with alpha, fp32 takes d up to 64 (LA_EUNSUPPORTED above: the fp32
 * tiles of the per-channel kernels exceed the LDS). */
typedef struct la_backward_args {
  int32_t B, H, N;   /* as the forward */
  int32_t d, dv;
  int32_t dtype;     /* la_dtype of q, k, v, o, grad_o and the gradients */
  int32_t fmap;      /* la_fmap of the forward */
  const void *q;     /* [B,H,N,d]  forward inputs */
  const void *k;     /* [B,H,N,d]  */
  const void *v;     /* [B,H,N,dv] */
  const void *o;     /* [B,H,N,dv] forward output */
  const float *den;  /* [B,H,N] forward denominators */
  const void *grad_o;/* [B,H,N,dv] dL/do */
  const float *gamma;/* [H] or NULL, as in the forward */
  const float *S_in; /* [B,H,d,dv] forward initial state; NULL = zeros */
  const float *z_in; /* [B,H,d]; NULL = zeros */
  const float *grad_S_out; /* [B,H,d,dv] dL/d(final state); NULL = zero */
  const float *grad_z_out; /* [B,H,d]; NULL = zero */
  void *grad_q;      /* [B,H,N,d]  outputs, dtype as q (required if N > 0) */
  void *grad_k;      /* [B,H,N,d]  */
  void *grad_v;      /* [B,H,N,dv] */
  float *grad_S_in;  /* [B,H,d,dv] dL/d(initial state); NULL = not written */
  float *grad_z_in;  /* [B,H,d]; NULL = not written */
  void *workspace;   /* device scratch of workspace_bytes, caller-owned;
                        4-byte aligned, 16-byte with conv_weight or alpha
                        (else LA_EINVAL) */
  size_t workspace_bytes;
  /* Optional (NULL = not used): the workspace of the la_prefill call that
   * produced o and den, left as that call wrote it, with this call's q, k,
   * v, gamma, S_in, z_in, fmap, convolution and no alpha; it holds the
   * state entering each segment of the forward (and with a convolution the
   * convolved q, k, v), which la_backward then reads (not written) instead
   * of recomputing it (the fp32 value-half passes recompute their own
   * segment states and read only the convolved inputs).
   * fwd_workspace_bytes below la_prefill_workspace_size of those
   * arguments: LA_EWORKSPACE; not 4-byte aligned (16-byte with
   * conv_weight): LA_EINVAL.  Any other contents give wrong gradients (not
   * detected).  Ignored when the forward needs no workspace. */
  const void *fwd_workspace;
  size_t fwd_workspace_bytes;
  /* The forward's short convolution (see la_prefill_args), or NULL: then
   * q, k, v are the raw inputs and the gradients are taken through the
   * convolution as well (the pages give no gradient formulas; the chain
   * rule: dL/dx_t = sum_j W_j dL/dy_(t+(w-1)-j), dL/dW_j = the sum over the
   * sequences and tokens of dL/dy_t times the input w-1-j tokens back). */
  const float *conv_weight;  /* [H, w, 2d+dv] filters */
  int32_t conv_width;        /* w, 1..4 with conv_weight; 0 without */
  const void *conv_in;       /* [B,H,w-1,2d+dv] the forward's conv cache before
                                the sequence (dtype of q), NULL = zeros */
  const void *grad_conv_out; /* [B,H,w-1,2d+dv] dL/d(the conv cache the forward
                                returned), dtype of q; NULL = zero */
  float *grad_conv_weight;   /* [H, w, 2d+dv] output (required with
                                conv_weight): summed over the batch */
  void *grad_conv_in;        /* [B,H,w-1,2d+dv] dL/d(conv_in), dtype of q;
                                NULL = not written */
  const float *alpha;        /* [B,H,N,d] the forward's per-key-channel decay,
                                or NULL; not with gamma (LA_EINVAL) */
  float *grad_alpha;         /* [B,H,N,d] dL/dalpha: required with alpha (if
                                N > 0), must be NULL without */
} la_backward_args;

/* Workspace bytes la_backward needs (0 when none); (size_t)-1 for invalid
 * sizes.  Reads only the sizes, the dtype, conv_width (with conv_weight set)
 * and whether alpha and fwd_workspace are NULL: with the forward's workspace given, the
 * forward's segment states (and convolved inputs) are read from it, so half
 * the state slots (and no copies of the inputs) are needed. */
size_t la_backward_workspace_size(const la_backward_args *args);

/* dq, dk, dv (and the initial-state gradient) of one LINEAR prefill. */
int la_backward(const la_backward_args *args, void *stream);

/* Backward of a gated-DELTA-rule prefill (training).  The pages motivate
 * parallel training ([WILA] section 8; [EAV] sections 8 and 10) but give no
 * gradient formulas; these are the reverse-mode derivatives of the rule
 * above, S_t = a_t (I - g_t k_t k_t^T) S_{t-1} + g_t k_t v_t^T,
 * o_t = S_t^T q_t (a_t = alpha_t, or 1 without a decay).  With the adjoint
 * Sh_t = dL/dS_t, the residual u_t = v_t - a_t S_{t-1}^T k_t and
 * w_t = Sh_t^T k_t:
 *   Sh_t = q_t do_t^T + a_(t+1) (I - g_(t+1) k_(t+1) k_(t+1)^T) Sh_(t+1)
 *   dq_t = S_t do_t,  dv_t = g_t w_t,  dg_t = w_t . u_t,
 *   dk_t = g_t Sh_t u_t - a_t g_t S_{t-1} w_t,
 *   dalpha_t = <Sh_t, S_{t-1}> - g_t (S_{t-1}^T k_t) . w_t,
 * and dL/d(initial state) = a_0 (I - g_0 k_0 k_0^T) Sh_0; computed chunk by
 * chunk (a forward pass over chunks for the states, a reverse pass for the
 * adjoint, then every chunk's gradients in parallel).  Inputs are the
 * forward's q, k, v, g, alpha and initial state, and dL/do (and optionally
 * dL/d(final state)); the forward's output is not needed.  bf16 only
 * (fp32: LA_EUNSUPPORTED). */
typedef struct la_delta_backward_args {
  int32_t B, H, N;   /* as the forward (each >= 0) */
  int32_t d, dv;     /* 1..128 */
  int32_t dtype;     /* la_dtype of q, k, v, grad_o and their gradients */
  const void *q;     /* [B,H,N,d]  forward inputs */
  const void *k;     /* [B,H,N,d]  */
  const void *v;     /* [B,H,N,dv] */
  const float *g;    /* [B,H,N] write gate */
  const float *alpha;/* [B,H,N] state decay, or NULL (none) */
  const float *S_in; /* [B,H,d,dv] forward initial state; NULL = zeros */
  const void *grad_o;/* [B,H,N,dv] dL/do */
  const float *grad_S_out; /* [B,H,d,dv] dL/d(final state); NULL = zero */
  void *grad_q;      /* [B,H,N,d]  outputs, dtype as q (required if N > 0) */
  void *grad_k;      /* [B,H,N,d]  */
  void *grad_v;      /* [B,H,N,dv] */
  float *grad_g;     /* [B,H,N] (required if N > 0) */
  float *grad_alpha; /* [B,H,N]: required with alpha, must be NULL without */
  float *grad_S_in;  /* [B,H,d,dv] dL/d(initial state); NULL = not written */
  void *workspace;   /* device scratch of workspace_bytes, caller-owned,
                        16-byte aligned (else LA_EINVAL) */
  size_t workspace_bytes;
  /* The forward's short convolution (see la_prefill_args), or NULL: then
   * q, k, v are the raw inputs and the gradients are taken through the
   * convolution as well (the pages give no gradient formulas; the chain
   * rule: dL/dx_t = sum_j W_j dL/dy_(t+(w-1)-j), dL/dW_j = the sum over the
   * sequences and tokens of dL/dy_t times the input w-1-j tokens back). */
  const float *conv_weight;  /* [H, w, 2d+dv] filters */
  int32_t conv_width;        /* w, 1..4 with conv_weight; 0 without */
  const void *conv_in;       /* [B,H,w-1,2d+dv] the forward's conv cache before
                                the sequence (dtype of q), NULL = zeros */
  const void *grad_conv_out; /* [B,H,w-1,2d+dv] dL/d(the conv cache the forward
                                returned), dtype of q; NULL = zero */
  float *grad_conv_weight;   /* [H, w, 2d+dv] output (required with
                                conv_weight): summed over the batch */
  void *grad_conv_in;        /* [B,H,w-1,2d+dv] dL/d(conv_in), dtype of q;
                                NULL = not written */
} la_delta_backward_args;

/* Workspace bytes la_delta_backward needs (0 when none); (size_t)-1 for
 * invalid sizes.  Reads only the sizes, the dtype and conv_width (with
 * conv_weight set). */
size_t la_delta_backward_workspace_size(const la_delta_backward_args *args);

/* dq, dk, dv, dg (and dalpha, the initial-state gradient) of one gated
 * delta prefill. */
int la_delta_backward(const la_delta_backward_args *args, void *stream);

/* One token per sequence against a persistent state updated in place. */
typedef struct la_decode_args {
  int32_t B, H;      /* sequences and heads (each >= 0) */
  int32_t d, dv;     /* 1..128 */
  int32_t dtype;     /* la_dtype of q, k, v and o */
  int32_t rule;      /* la_rule */
  int32_t fmap;      /* la_fmap (DELTA: IDENTITY only) */
  const void *q;     /* [B,H,d]  */
  const void *k;     /* [B,H,d]  */
  const void *v;     /* [B,H,dv] */
  const float *gamma;/* LINEAR: [H] or NULL (=1).  DELTA: must be NULL. */
  const float *g;    /* DELTA: [B,H] write gate (required). LINEAR: NULL. */
  const float *alpha;/* State decay, or NULL (= 1).  DELTA: [B,H].
                        LINEAR: [B,H,d] per key channel (not with gamma). */
  const float *conv_weight; /* [H, w, 2d+dv] short-convolution filters,
                        or NULL (either rule). */
  int32_t conv_width;/* w, 1..4 with conv_weight; 0 without */
  void *conv_cache;  /* [B,H,w-1,2d+dv] conv cache, dtype as q, read and
                        shifted in place by one token (required for w > 1) */
  float eps;         /* LINEAR: >= 0 */
  float *S;          /* [B,H,d,dv] fp32, read and overwritten in place */
  float *z;          /* LINEAR: [B,H,d] fp32 in place (required).
                        DELTA: must be NULL. */
  void *o;           /* [B,H,dv] output, dtype as q */
} la_decode_args;

/* One decode step ([LIO3] 'recurrent form': one read and one write of the
 * state per token).  S (and z, conv_cache) must not overlap q, k, v or o,
 * or one another. */
int la_decode_step(const la_decode_args *args, void *stream);

/* Zero-fill a state: S [B,H,d,dv] and, if z is not NULL, z [B,H,d]
 * ([LIO3] 'implementation': the state starts as zeros).  Uses a fill
 * kernel (no memset node), so it may be captured in a HIP graph. */
int la_state_init(float *S, float *z, int32_t B, int32_t H, int32_t d,
                  int32_t dv, void *stream);

/* Static description of a status code (never NULL). */
const char *la_status_str(int status);

/* Kernel timing for benchmarks and tracing (not part of the method).
 * While enabled, every kernel the library launches gets a pair of HIP
 * events that the dispatch itself stamps when the kernel starts and ends
 * (hipExtLaunchKernel; no host synchronisation).  la_profile_collect() waits for the
 * recorded events, writes up to `max` records (oldest first) and clears the
 * log; it returns the number of records written, or -1 on a HIP error.
 * Records past an internal limit of 65536 are dropped.  Kernel names are
 * static strings.  Enabling/disabling clears the log.  Not meant to be
 * toggled while another thread is launching. */
typedef struct la_kernel_time {
  const char *name; /* kernel name (static storage) */
  float ms;         /* kernel duration (start to end of the dispatch) */
} la_kernel_time;
int la_profile_enable(int on);
int la_profile_collect(la_kernel_time *out, int max);

/* ABI version: bumped whenever a struct above changes layout. */
int32_t la_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
