/*
 * ssm_scan.h -- C ABI of the selective-SSM scan library for AMD MI355X (gfx950).
 *
 * The library computes the selective state-space scan of Mamba (Gu & Dao,
 * "Mamba: Linear-Time Sequence Modeling with Selective State Spaces", arXiv
 * 2312.00752).  The pages this follows are the paper's reading guide on
 * xyznot.com and the mamba-minimal news page on ja.news.hada.io:
 *
 *   per batch row b, channel d and state index n, for t = 0 .. L-1
 *     s_t       = delta[b,t,d] + delta_bias[d]
 *     dt_t      = softplus(s_t) if delta_softplus else s_t
 *                 (reading guide, "Seçim Mekanizması (S6)": the step size is
 *                 softplus of a parameter plus an input-dependent term)
 *     dA        = exp(dt_t * A[d,n])       (zero-order hold of A, "Yöntem")
 *     dBu       = dt_t * B[b,t,n] * u[b,t,d]
 *                 (the deltaB_u term of the sequential loop quoted on the
 *                 mamba-minimal page; first-order form of the ZOH input term)
 *     h[n]      = dA * h[n] + dBu          (discrete recurrence, "Yöntem")
 *     y[b,t,d]  = (sum_n C[b,t,n] * h[n] + D[d] * u[b,t,d]) * silu(z[b,t,d])
 *                 (output y = C h, "Yöntem"; D skip and the multiplicative
 *                 SiLU gate of the Mamba block, "Temel Fikirler")
 *
 * The expanded (B,L,D,N) state never exists in device memory: it lives in
 * registers, and only the contracted (B,L,D) output is written ("Donanım
 * Duyarlı Durum Genişletme" section of the reading guide).
 *
 * Conventions shared by every entry point:
 *   - All tensors are dense, row-major, contiguous, in device memory.
 *     (B,L,D) tensors: u, delta, z, y, dy, du, ddelta, dz.
 *     (B,L,N) tensors: Bmat, Cmat, dB, dC.        (D,N): A, dA.
 *     (D): Dskip, delta_bias, dD, ddelta_bias.    (B,D,N): h0, h_final, dh_final, dh0, state.
 *   - io_dtype (SSM_F32 or SSM_BF16) is the storage type of u, delta, z,
 *     Bmat, Cmat, y and of their gradients.  A, Dskip, delta_bias, every
 *     state and dA, dD, ddelta_bias, dh0 are always fp32.  Arithmetic is fp32;
 *     bf16 outputs are rounded to nearest even.
 *   - Every pointer must be 16-byte aligned (ssm_state_update relaxes this,
 *     see there); dim must be a multiple of 8;
 *     dstate must be 1, 2, 4, 8 or 16; batch, seqlen, dim >= 1; batch <= 2^31 - 1;
 *     dim <= 2^36 (the channel tiles of a batch row are a grid dimension).
 *   - The caller owns all memory.  The library never allocates, frees or
 *     synchronises device memory; it enqueues kernels on hip_stream (a
 *     hipStream_t; NULL = the default stream) and returns at once.
 *   - Return value: SSM_OK or a positive ssm_status.  All arguments are
 *     validated before anything is enqueued, so on error nothing is written.
 *     ssm_last_error() gives a message for the last failing call on the
 *     calling thread.  NaN and Inf in the inputs propagate; they are not
 *     errors.
 *   - Output buffers must not overlap input buffers (except state in
 *     ssm_state_update, which is updated in place by design).
 */
#ifndef SSM_SCAN_H_
#define SSM_SCAN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_SCAN_ABI_VERSION 4

typedef enum ssm_status {
  SSM_OK = 0,
  SSM_ERR_NULL_ARG = 1,    /* a required pointer is NULL, or an optional pair is inconsistent */
  SSM_ERR_BAD_SHAPE = 2,   /* a size is < 1 (or would overflow 64-bit offsets) */
  SSM_ERR_UNSUPPORTED = 3, /* dstate not in {1,2,4,8,16}, dim % 8 != 0, batch >= 2^31, dim > 2^36,
                              unknown io_dtype */
  SSM_ERR_ALIGNMENT = 4,   /* a pointer is not 16-byte aligned */
  SSM_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the size query returns */
  SSM_ERR_HIP = 6          /* the HIP runtime reported an error while enqueuing */
} ssm_status;

typedef enum ssm_dtype { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/*
 * Option bits of the *_ex entry points (0 = the definition above).
 *
 * SSM_FLAG_ZOH: the exact zero-order-hold input term of the reading guide's
 *   "Yöntem" discretisation, Bbar = (dt A)^-1 (exp(dt A) - 1) dt B, so that
 *   dBu = expm1(dt A) / A * B * u (= dt B u in the limit A -> 0) instead of
 *   dt * B * u.  Forward, backward and single-token update.
 * SSM_FLAG_REVERSE: the recurrence runs from the last step to the first,
 *   h_t = exp(dt_t A) h_{t+1} + dBu_t; h0 is the state before step L-1,
 *   h_final the state after step 0, and chunk slot k the state before scan
 *   step k*T (time L-1-k*T).  This is the second direction of a bidirectional
 *   mixer (Hydra, on the zenn.dev reading list); see SSM_FLAG_ACCUMULATE.
 *   Forward and backward.
 * SSM_FLAG_DELTA_PER_TOKEN: delta is (B, L), one raw step size per token
 *   shared by every channel, plus the per-channel delta_bias (the reading
 *   guide's "Seçim Mekanizması (S6)" delta equation broadcasts one value over
 *   D).  ddelta is then (B, L): the sum of the per-channel gradients.
 *   Forward and backward.
 * SSM_FLAG_ACCUMULATE: forward only; y += scan output instead of y = scan
 *   output (y is read, so it must hold valid data).  A forward scan followed
 *   by a reverse scan with this flag sums both directions.
 */
#define SSM_FLAG_ZOH 1
#define SSM_FLAG_REVERSE 2
#define SSM_FLAG_DELTA_PER_TOKEN 4
#define SSM_FLAG_ACCUMULATE 8

/* SSM_SCAN_ABI_VERSION of the built library. */
int ssm_abi_version(void);

/* Static description of a status code ("ok", "null argument", ...). */
const char *ssm_status_string(int status);

/* Message of the last failing call on the calling thread ("" if none).  The
 * pointer stays valid until the next library call on that thread. */
const char *ssm_last_error(void);

/* Number of time steps T between two saved chunk-boundary states (32). */
int64_t ssm_scan_chunk_len(void);

/* Bytes of the chunk_states buffer: batch * ceil(seqlen/T) * dim * dstate * 4.
 * Layout (B, K, N, D) fp32 (channels fastest), K = ceil(seqlen/T); slot k
 * holds the state just before step k*T (slot 0 is h0, or zeros).  Returns -1
 * on invalid sizes. */
int64_t ssm_scan_chunk_states_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/* Device workspace the forward scan needs for these sizes (may be 0; then
 * workspace may be NULL).  Returns -1 on invalid sizes. */
int64_t ssm_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                     int io_dtype);

/*
 * How ssm_scan_fwd (and its _ex and _conv forms) would run these sizes on the
 * current device: the kernel, the channels each workgroup owns, and the
 * sequence split.  A host-side query: it launches nothing and touches no
 * device memory (it reads the device's compute-unit count once per process;
 * without a device it assumes 256).  Tests use it to show which kernel
 * variant a shape reaches.  conv_width is 0 for the plain scan, else the
 * width of the fused convolution.  Returns SSM_OK and fills *plan, or an
 * error status as for the forward itself (nothing written on error).
 */
typedef struct ssm_fwd_plan {
  int32_t kernel;        /* 0: all-purpose kernel (every phase on every wave);
                            1: wave-specialised kernel (16 states: recurrence
                               waves and service waves) */
  int32_t tile_channels; /* channels per workgroup: 16, 32, 64 or 80 */
  int64_t segments;      /* sequence segments (1 = no split) */
  int64_t segment_len;   /* steps per segment (0 = no split) */
  int64_t first_pass_len; /* steps per piece of a split's first pass, which
                             finds the end state of every segment but the
                             last in segment_len / first_pass_len pieces
                             (0 = no split) */
} ssm_fwd_plan;

int ssm_scan_fwd_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                      int flags, int conv_width, ssm_fwd_plan *plan);

/*
 * Forward selective scan (the recurrence above over all L steps).
 *
 * Inputs:  u, delta (raw step size, before bias and softplus), z (optional
 *          gate; NULL = no gate), Bmat, Cmat in io_dtype; A (D,N), Dskip
 *          (optional, NULL = 0), delta_bias (optional, NULL = 0) fp32;
 *          delta_softplus (0/1); h0 (optional initial state, NULL = zeros).
 * Outputs: y (B,L,D) io_dtype; h_final (optional, NULL = not wanted) the
 *          state after the last step; chunk_states (optional, NULL = not
 *          wanted) the states at chunk boundaries, needed by ssm_scan_bwd.
 * Workspace: ssm_scan_fwd_workspace_bytes() bytes of device memory, contents
 *          undefined on entry and exit.
 * Errors:  SSM_ERR_* as in the conventions; nothing is enqueued on error.
 */
int ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                 const void *u, const void *delta, const float *A, const void *Bmat,
                 const void *Cmat, const float *Dskip, const void *z, const float *delta_bias,
                 int delta_softplus, const float *h0, float *h_final, void *y,
                 float *chunk_states, void *workspace, int64_t workspace_bytes,
                 void *hip_stream);

/* ssm_scan_fwd with option bits (SSM_FLAG_*; all four apply).  Unknown bits
 * return SSM_ERR_UNSUPPORTED.  flags = 0 is exactly ssm_scan_fwd.  The
 * workspace size does not depend on the flags. */
int ssm_scan_fwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                    const void *u, const void *delta, const float *A, const void *Bmat,
                    const void *Cmat, const float *Dskip, const void *z, const float *delta_bias,
                    int delta_softplus, const float *h0, float *h_final, void *y,
                    float *chunk_states, void *workspace, int64_t workspace_bytes,
                    void *hip_stream, int flags);

/*
 * ssm_scan_fwd_ex without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It allocates nothing: the workspace a
 * sequence split needs (ssm_scan_fwd_workspace_bytes) lives in a static
 * device array of SSM_NOALLOC_SCRATCH_BYTES that the library's code object
 * holds on every device it runs on until the process ends.  Sizes whose
 * workspace exceeds that return SSM_ERR_WORKSPACE before anything is enqueued.
 * The array is shared by every call on one device and keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap on one
 * device (different streams, or host threads) race and must be serialised by
 * the caller.  Arguments, outputs and errors otherwise as ssm_scan_fwd_ex;
 * the result is identical to it.
 */
#define SSM_NOALLOC_SCRATCH_BYTES (16 << 20)

int ssm_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                         const void *u, const void *delta, const float *A, const void *Bmat,
                         const void *Cmat, const float *Dskip, const void *z,
                         const float *delta_bias, int delta_softplus, const float *h0,
                         float *h_final, void *y, float *chunk_states, void *hip_stream, int flags);

/* Device workspace ssm_scan_bwd needs for these sizes.  -1 on invalid sizes. */
int64_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                     int io_dtype);

/*
 * Backward of ssm_scan_fwd: gradients of a scalar loss given dy = dLoss/dy
 * and (optionally) dh_final = dLoss/dh_final.  States inside a chunk are
 * recomputed from chunk_states (written by ssm_scan_fwd with the same
 * inputs) instead of being read from memory (reading guide, "Donanım Duyarlı
 * Durum Genişletme": intermediate states are recomputed in the backward
 * pass).
 *
 * Inputs:  the forward's inputs (same meaning, same pointers allowed),
 *          chunk_states (required), dy (B,L,D) io_dtype, dh_final (optional).
 * Outputs (all overwritten, never accumulated):
 *          du, ddelta (w.r.t. the raw delta), dz (required iff z != NULL)
 *          (B,L,D) io_dtype; dB, dC (B,L,N) io_dtype; dA (D,N) fp32;
 *          dD (D) fp32, required iff Dskip != NULL; ddelta_bias (D) fp32,
 *          optional; dh0 (B,D,N) fp32, optional.
 * Workspace: ssm_scan_bwd_workspace_bytes() bytes, contents undefined.
 * Sums over channels and time are fp32 in a fixed order: repeated calls give
 * bit-identical results.
 */
int ssm_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                 const void *u, const void *delta, const float *A, const void *Bmat,
                 const void *Cmat, const float *Dskip, const void *z, const float *delta_bias,
                 int delta_softplus, const float *h0, const float *chunk_states, const void *dy,
                 const float *dh_final, void *du, void *ddelta, float *dA, void *dB, void *dC,
                 float *dD, void *dz, float *ddelta_bias, float *dh0, void *workspace,
                 int64_t workspace_bytes, void *hip_stream);

/* ssm_scan_bwd with option bits: SSM_FLAG_ZOH, SSM_FLAG_REVERSE and
 * SSM_FLAG_DELTA_PER_TOKEN, which must match the forward that wrote
 * chunk_states (SSM_FLAG_ACCUMULATE and unknown bits return
 * SSM_ERR_UNSUPPORTED).  With SSM_FLAG_DELTA_PER_TOKEN, delta and ddelta are
 * (B, L).  flags = 0 is exactly ssm_scan_bwd. */
int ssm_scan_bwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                    const void *u, const void *delta, const float *A, const void *Bmat,
                    const void *Cmat, const float *Dskip, const void *z, const float *delta_bias,
                    int delta_softplus, const float *h0, const float *chunk_states, const void *dy,
                    const float *dh_final, void *du, void *ddelta, float *dA, void *dB, void *dC,
                    float *dD, void *dz, float *ddelta_bias, float *dh0, void *workspace,
                    int64_t workspace_bytes, void *hip_stream, int flags);

/*
 * The scan fed by the causal depthwise convolution of the Mamba block (the
 * Italian overview article on nisoo.com, "Iniziare con Mamba": the block puts a
 * causal Conv1d in front of the selective SSM; reading guide, "Temel
 * terimler", Mamba block), fused so that u never goes to memory:
 *   pre[b,t,d] = conv_b[d] + sum_{k<K} conv_w[d,k] x[b, t-(K-1)+k, d]
 *                (x = 0 before the first step; tap K-1 multiplies the
 *                current step), u = silu(pre) = pre * sigmoid(pre),
 * then exactly ssm_scan_fwd_ex on u.  x is (B,L,D) in io_dtype; conv_w is
 * (D,K) fp32 with K = conv_width in 1..4; conv_b (D) fp32 is optional.
 * flags: SSM_FLAG_ZOH, SSM_FLAG_DELTA_PER_TOKEN, SSM_FLAG_ACCUMULATE
 * (SSM_FLAG_REVERSE is rejected: the convolution runs forward in time).
 * Workspace as for ssm_scan_fwd.
 */
int ssm_scan_fwd_conv(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                      const void *x, const float *conv_w, const float *conv_b, int conv_width,
                      const void *delta, const float *A, const void *Bmat, const void *Cmat,
                      const float *Dskip, const void *z, const float *delta_bias,
                      int delta_softplus, const float *h0, float *h_final, void *y,
                      float *chunk_states, void *workspace, int64_t workspace_bytes,
                      void *hip_stream, int flags);

/* Device workspace ssm_scan_bwd_conv needs.  -1 on invalid sizes. */
int64_t ssm_scan_bwd_conv_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim,
                                          int64_t dstate, int io_dtype);

/*
 * Backward of ssm_scan_fwd_conv.  u is recomputed from x (the convolution's
 * pre-activation is written to the workspace first).  Outputs as for
 * ssm_scan_bwd_ex with du replaced by dx (B,L,D) io_dtype, plus dconv_w (D,K)
 * fp32 and dconv_b (D) fp32 (required iff conv_b != NULL), all overwritten:
 *   g = dLoss/du * silu'(pre),  dx[b,t,d] = sum_k conv_w[d,k] g[b, t+(K-1)-k, d],
 *   dconv_w[d,k] = sum_{b,t} x[b, t-(K-1)+k, d] g[b,t,d],  dconv_b[d] = sum_{b,t} g.
 * flags: SSM_FLAG_ZOH and SSM_FLAG_DELTA_PER_TOKEN, matching the forward.
 * Workspace: ssm_scan_bwd_conv_workspace_bytes() bytes.  Sums are in a fixed
 * order (deterministic).
 */
int ssm_scan_bwd_conv(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                      const void *x, const float *conv_w, const float *conv_b, int conv_width,
                      const void *delta, const float *A, const void *Bmat, const void *Cmat,
                      const float *Dskip, const void *z, const float *delta_bias,
                      int delta_softplus, const float *h0, const float *chunk_states,
                      const void *dy, const float *dh_final, void *dx, float *dconv_w,
                      float *dconv_b, void *ddelta, float *dA, void *dB, void *dC, float *dD,
                      void *dz, float *ddelta_bias, float *dh0, void *workspace,
                      int64_t workspace_bytes, void *hip_stream, int flags);

/*
 * Scan of affine maps along rows (fp32, row-major (rows, len), device memory):
 *   s = h0[r] (0 if h0 is NULL); for i in scan order: s = a[r,i] * s + b[r,i];
 *   h[r,i] = s.
 * Scan order is i = 0 .. len-1, or len-1 .. 0 if reverse = 1.  Every step of
 * the recurrence is such a map (reading guide, "Yöntem": the new state is the
 * discretised A times the old state plus the discretised input), and because
 * the maps compose associatively -- (a1, b1) then (a2, b2) is (a1 a2,
 * a2 b1 + b2) -- the scan runs in parallel: one wave per row, 64 positions at
 * a time with a wave-wide associative scan (DPP cross-lane moves), the state
 * carried between pieces.  The library folds the segments of a split sequence
 * with the same primitive; this entry point exposes it, for example to fold
 * the segment aggregates of a sequence sharded over several devices.  Results
 * equal the sequential loop up to the rounding of the different association
 * (exactly, when every product and sum is exact in fp32).
 * Pointers need 4-byte alignment; h may be the same array as a or b.  Errors:
 * rows or len < 1 (SSM_ERR_BAD_SHAPE), rows > 4 * (2^31 - 1) or reverse not 0
 * or 1 (SSM_ERR_UNSUPPORTED), a, b or h NULL (SSM_ERR_NULL_ARG); nothing is
 * enqueued on error.
 */
int ssm_affine_scan(int64_t rows, int64_t len, const float *a, const float *b, const float *h0,
                    float *h, int reverse, void *hip_stream);

/*
 * One decode step (reading guide, "Sorular", the question on KV caches: the
 * model keeps a fixed D x N state per layer and advances it one token at a
 * time).  state (B,D,N) fp32 is read once and overwritten in place with the
 * new state; u, delta, z, y are (B,D) and Bmat, Cmat are (B,N) in io_dtype.
 * Same arithmetic as one step of ssm_scan_fwd.  Alignment: state and A must be
 * 16-byte aligned; the other pointers only need their element alignment.
 */
int ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, int io_dtype, float *state,
                     const void *u, const void *delta, const float *A, const void *Bmat,
                     const void *Cmat, const float *Dskip, const void *z,
                     const float *delta_bias, int delta_softplus, void *y, void *hip_stream);

/* ssm_state_update with option bits: only SSM_FLAG_ZOH applies to one token
 * (other bits return SSM_ERR_UNSUPPORTED).  flags = 0 is exactly
 * ssm_state_update. */
int ssm_state_update_ex(int64_t batch, int64_t dim, int64_t dstate, int io_dtype, float *state,
                        const void *u, const void *delta, const float *A, const void *Bmat,
                        const void *Cmat, const float *Dskip, const void *z,
                        const float *delta_bias, int delta_softplus, void *y, void *hip_stream,
                        int flags);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H_ */
