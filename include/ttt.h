/*
 * ttt.h -- C ABI of the MI355X (gfx950) TTT-layer forward scan, its
 * streaming (decode) step and its backward pass.
 *
 * The method (arXiv 2407.04620, "Learning to (Learn at Test Time): RNNs with
 * Expressive Hidden States"; summarised in the dmarx.github.io record
 * LIT-801, "Key takeaways" items 1, 2 and 5, and in the codewithpapers.app
 * record's "abstract"): a sequence layer whose hidden state is the weights S
 * of an inner model f.  For each (batch, head) unit and each token t,
 *     loss    l(S; k, v) = || f(k; S) - v ||^2                 (item 2)
 *     update  S_t = S_{t-1} - eta_t * grad l(S_{t-1}; k_t, v_t)  (item 1)
 *     output  z_t = f(q_t; S_t)                                (item 1)
 * with mini-batch inner gradient descent (item 5): the gradients of the
 * tokens of one mini-batch of b tokens are all taken at the state held when
 * the mini-batch began, and the state absorbs them token by token, so z_t
 * sees the updates of tokens s <= t.  A last partial mini-batch (T mod b
 * != 0) is one step on its tokens.  Inner models (abstract; item 5):
 *     TTT-Linear  f(x) = x + LN(x W)                        state W  [d,d]
 *     TTT-MLP     f(x) = x + LN(GELU(x W1 + b1) W2 + b2)    state W1 [d,m],
 *                                                  b1 [m], W2 [m,d], b2 [d]
 * LN normalises the d features of one token (biased variance, epsilon
 * ln_eps) and applies the per-head gamma/beta, which are parameters, not
 * state.  GELU is the exact erf form.  The loss is the squared Euclidean
 * norm summed over the d outputs; eta_t is used exactly as given.
 * TTT_NO_LN and TTT_NO_RESIDUAL drop the LN or the residual (both: the
 * linear model of Theorem 1, item 3).
 *
 * Conventions shared by every entry point
 *  - Pointers q, k, v, eta, states, gamma, beta, z, the *_out buffers and
 *    workspaces are DEVICE pointers (HIP global memory of the current
 *    device), owned by the caller.  The library allocates no memory and
 *    keeps no global mutable state (one exception: the per-device address
 *    of the fixed scratch array of ttt_linear_forward_split_noalloc, looked
 *    up once per device under a lock); calls are thread-safe and reentrant.
 *  - Layout: contiguous, row-major, feature dimension fastest.
 *      q, k, v, z  [B,H,T,d] of io_dtype     eta  [B,H,T] fp32
 *      gamma, beta [H,d] fp32 (not read with TTT_NO_LN; may be NULL then)
 *      initial state: [H,...] fp32 shared across the batch, or [B,H,...]
 *      when state0_per_batch = 1.  Final state: [B,H,...] fp32.
 *  - Execution is asynchronous on hip_stream (NULL = the default stream).
 *    Outputs are valid once the caller synchronises that stream.
 *  - Errors: argument errors are detected before anything is launched and
 *    nothing is written.  A launch failure returns TTT_ERR_DEVICE.  Faults
 *    during execution surface at the caller's next synchronisation.  No C++
 *    exception crosses this boundary.
 *  - Aliasing: z must not overlap q, k, v or eta (TTT_ERR_ALIAS).  A final
 *    state buffer may equal the matching initial-state buffer only when
 *    state0_per_batch = 1 (in-place resume; each unit reads its whole state
 *    before it writes any of it); any other overlap between outputs and
 *    inputs is TTT_ERR_ALIAS.
 *  - Resume: the final state of a call started with the last tokens of a
 *    sequence is the initial state (state0_per_batch = 1) of a call on the
 *    continuation; this is exact when the first call's T is a multiple of
 *    the mini-batch size.
 */
#ifndef TTT_H
#define TTT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTT_ABI_VERSION 11

typedef enum {
  TTT_OK = 0,
  TTT_ERR_NULL = 1,         /* a required pointer is NULL */
  TTT_ERR_SHAPE = 2,        /* B, H, T, d, mini_batch or hidden out of range, or a
                               workspace smaller than its query returned */
  TTT_ERR_UNSUPPORTED = 3,  /* valid for the method, not built for gfx950 (or a split
                               launch on more units than half the compute units) */
  TTT_ERR_ALIAS = 4,        /* forbidden overlap between buffers */
  TTT_ERR_DEVICE = 5,       /* HIP reported an error at launch */
  TTT_ERR_ARG = 6,          /* bad dtype, flag or epsilon, or a misaligned workspace */
  TTT_ERR_TOO_LARGE = 7     /* the problem needs more scratch than the fixed array of
                               ttt_linear_forward_split_noalloc holds */
} ttt_status;

typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;

enum {
  TTT_NO_LN = 1u << 0,        /* f(x) = [x +] g(x) */
  TTT_NO_RESIDUAL = 1u << 1,  /* f(x) = [LN](g(x)) */
  TTT_BASES_SAVED = 1u << 2   /* ttt_linear_backward only: see there */
};

typedef struct {
  int32_t B, H, T, d;        /* B, H >= 1; 1 <= T <= 4194304; d == 64 on gfx950 */
  int32_t mini_batch;        /* b: Linear 16*n (n >= 1; b >= T allowed); MLP 16 */
  int32_t io_dtype;          /* ttt_dtype of q, k, v and z */
  uint32_t flags;            /* TTT_NO_LN | TTT_NO_RESIDUAL */
  float ln_eps;              /* LN epsilon, >= 0 (the workloads use 1e-6) */
  int32_t state0_per_batch;  /* 0: initial state [H,...]; 1: [B,H,...] */
} ttt_params;

/*
 * TTT-Linear forward scan.
 *   w0     [H,d,d] (or [B,H,d,d]) fp32, input row index first: h = x W.
 *   z      [B,H,T,d] io_dtype, written for every token.
 *   w_out  [B,H,d,d] fp32 final state, or NULL to skip it.
 * Supported: d = 64, mini_batch a positive multiple of 16 (values >= T
 * give batch GD over the causal prefix), both io dtypes, any flags.
 * gfx950 kernel: one 768-thread workgroup per (batch, head) unit; the state
 * stays in registers across the whole sequence.
 */
ttt_status ttt_linear_forward(const ttt_params* p,
                              const void* q, const void* k, const void* v,
                              const float* eta, const float* w0,
                              const float* ln_gamma, const float* ln_beta,
                              void* z, float* w_out, void* hip_stream);

/*
 * Bytes of device workspace that ttt_linear_forward_split needs for these
 * parameters: 256 bytes per unit plus 256, and 6 KB per unit and 16-token
 * tile (0 if p fails the common checks).
 */
uint64_t ttt_linear_split_workspace_bytes(const ttt_params* p);

/*
 * TTT-Linear forward scan, same method, arguments and results as
 * ttt_linear_forward (bit for bit; but no in-place resume: w_out == w0 is
 * TTT_ERR_ALIAS here), on two workgroups per (batch, head)
 * unit: one runs the serial part of the scan (the gradient of every
 * 16-token tile) and streams each tile's gradient through `workspace` to
 * the other, on another compute unit, which replays the state updates and
 * forms z.  Unit count B*H at most half the device's compute units
 * (TTT_ERR_UNSUPPORTED otherwise; use ttt_linear_forward).
 *   workspace  device memory, 256-byte aligned, at least
 *              ttt_linear_split_workspace_bytes(p) bytes, owned by the
 *              caller, overlapping no other argument (TTT_ERR_SHAPE /
 *              TTT_ERR_ARG / TTT_ERR_ALIAS).  Its contents need no
 *              initialisation and are scratch after the call; it serves one
 *              call at a time (calls that overlap in time must use distinct
 *              workspaces).
 * The launch is two kernels on hip_stream (a fill of the workspace's
 * counters, then the scan).  Should the second workgroup of a unit wait
 * for the first for seconds (the two not resident together), it gives up
 * and writes NaN to that unit's z instead of hanging; the final state is
 * always correct.
 */
ttt_status ttt_linear_forward_split(const ttt_params* p,
                                    const void* q, const void* k, const void* v,
                                    const float* eta, const float* w0,
                                    const float* ln_gamma, const float* ln_beta,
                                    void* z, float* w_out,
                                    void* workspace, uint64_t workspace_bytes,
                                    void* hip_stream);

/*
 * ttt_linear_forward_split without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same method, arguments, results (bit for bit) and restrictions as
 * ttt_linear_forward_split; the gradient stream and the publication
 * counters live in a fixed array in the library's device code instead of a
 * caller workspace:
 *  - its size is TTT_NOALLOC_SCRATCH_BYTES (128 MiB) per device; a problem
 *    whose ttt_linear_split_workspace_bytes exceeds it (256 bytes per unit,
 *    256, and 6 KB per unit and 16-token tile; e.g. B*H = 32 units up to
 *    T = 10912) returns TTT_ERR_TOO_LARGE before anything runs;
 *  - every GPU the library runs on holds its own copy of the array (device
 *    memory taken when the library's code is loaded on that device, kept
 *    until the process ends); its address is looked up once per device, on
 *    the first call with that device current;
 *  - every call on one device shares that device's array, and the counters
 *    are cleared by the call's own fill kernel: calls on one device must not
 *    overlap in time (enqueue them on one stream, or order the streams);
 *    overlapping calls race and give wrong results.
 * No hipMalloc, hipFree or allocating library routine is called.
 */
#define TTT_NOALLOC_SCRATCH_BYTES (128ull << 20)
ttt_status ttt_linear_forward_split_noalloc(const ttt_params* p,
                                            const void* q, const void* k, const void* v,
                                            const float* eta, const float* w0,
                                            const float* ln_gamma, const float* ln_beta,
                                            void* z, float* w_out, void* hip_stream);

/*
 * One token of the TTT-Linear scan per (batch, head) unit: the streaming
 * (decode) step.  Within a mini-batch every gradient is taken at the state
 * the mini-batch started from (its base), so a stream carries the state W,
 * the base W_base and the position `pos` (0 <= pos < mini_batch) of the next
 * token in its mini-batch.  The step takes the gradient at
 * base = (pos == 0 ? W : W_base), updates W <- W - eta_t * gradient, writes
 * z_t = f(q_t; W) and, when pos == 0, stores base into W_base.  Calling it
 * for t = 0, 1, ... with pos = t mod mini_batch, starting from W = W0,
 * reproduces ttt_linear_forward (the LIT-801 record, "Key takeaways" items
 * 1, 2 and 5).
 *   p        T must be 1; mini_batch any b >= 1; state0_per_batch unused.
 *   q, k, v  [B,H,d] io_dtype;  eta [B,H] fp32;  z [B,H,d] io_dtype (out).
 *   w        [B,H,d,d] fp32, read and written (in place).
 *   w_base   [B,H,d,d] fp32: read when pos > 0, written when pos == 0.
 * w, w_base and z overlap nothing else (TTT_ERR_ALIAS); pos out of range is
 * TTT_ERR_ARG.  gfx950 kernel: one 256-thread workgroup per unit, fp32
 * arithmetic; bound by moving the state (about 48 KB per unit and token).
 */
ttt_status ttt_linear_decode_step(const ttt_params* p, int32_t pos,
                                  const void* q, const void* k, const void* v,
                                  const float* eta, float* w, float* w_base,
                                  const float* ln_gamma, const float* ln_beta,
                                  void* z, void* hip_stream);

/*
 * The streaming step of ttt_linear_decode_step with a compact pending
 * state: the same tokens, the same z (up to rounding order).  Within a
 * mini-batch the state after the tokens s < pos is
 *     W = w_base + sum_{s<pos} k_s^T u_s,    u_s = -eta_s * gradient_s,
 * so the stream carries the base and the mini-batch's rows instead of W:
 *   w_base  [B,H,d,d] fp32, read; at pos == 0 first replaced by
 *           w_base + sum over all mini_batch history slots (the previous
 *           mini-batch; zeros at the start of a stream).
 *   hist    [B,H,mini_batch,2,d] fp32: slot s holds k_s then u_s; slot
 *           pos is written.  Zero it when a stream starts.
 * About 22 KB move per unit and token for mini_batch = 16 (48 KB for the
 * (W, W_base) form).  The final state of a ttt_linear_forward over a whole
 * number of mini-batches starts a stream as w_base with a zero history.
 *   p   T must be 1; mini_batch at most 64 (TTT_ERR_UNSUPPORTED).
 * Other arguments, aliasing and errors as ttt_linear_decode_step.
 */
ttt_status ttt_linear_decode_step_compact(const ttt_params* p, int32_t pos,
                                          const void* q, const void* k, const void* v,
                                          const float* eta, float* w_base, float* hist,
                                          const float* ln_gamma, const float* ln_beta,
                                          void* z, void* hip_stream);

/*
 * TTT-Linear forward scan for training: ttt_linear_forward (same arguments
 * and results, bit for bit, on the one-workgroup launch) that also stores
 * the base of every 16-token mini-batch -- the state the mini-batch's
 * gradients are taken at, which the forward holds anyway -- into
 * `workspace`, for a later ttt_linear_backward with TTT_BASES_SAVED.
 *   workspace  as for ttt_linear_backward (at least
 *              ttt_linear_backward_workspace_bytes(p) bytes, 256-byte
 *              aligned, overlapping no other argument); its base region is
 *              written, the rest untouched.
 * Supported: mini_batch = 16 (else TTT_ERR_UNSUPPORTED).  Adds 16 KB of
 * stores per unit and mini-batch to the forward.
 */
ttt_status ttt_linear_forward_save(const ttt_params* p,
                                   const void* q, const void* k, const void* v,
                                   const float* eta, const float* w0,
                                   const float* ln_gamma, const float* ln_beta,
                                   void* z, float* w_out,
                                   void* workspace, uint64_t workspace_bytes,
                                   void* hip_stream);

/*
 * Bytes of device workspace that ttt_linear_backward needs for these
 * parameters: 16 KB per unit and 16-token tile (the state at every tile's
 * start), plus 16 KB + 512 bytes per unit, rounded up to 256 bytes; with
 * mini_batch = 16 another 15,104 bytes per unit and tile (the records
 * that the front half of each tile, computed for all tiles at once, leaves
 * for the reverse walk) (0 if p fails the common checks).  About 2 GB for
 * B = 4, H = 32, T = 8192 with 16-token mini-batches.
 */
uint64_t ttt_linear_backward_workspace_bytes(const ttt_params* p);

/*
 * Backward pass of the TTT-Linear forward scan: the vector-Jacobian product
 * that training needs, since the outer loop trains the projections behind
 * q, k and v, the initial state and the per-token learning rate (the
 * LIT-801 record, "Key takeaways" item 2), and the LN parameters of f.
 * For cotangents dz (and dw_final on the final state) it writes the
 * gradients of  L = sum_t <dz_t, z_t> + <dw_final, W_T>  with respect to
 * every input of ttt_linear_forward (same p, same inputs).
 *   dz        [B,H,T,d] io_dtype.
 *   dw_final  [B,H,d,d] fp32, or NULL for zero.
 *   dq, dk, dv  [B,H,T,d] io_dtype (out; rounded once from fp32).
 *   deta      [B,H,T] fp32 (out).
 *   dw0       w0's shape, fp32 (out): summed over the batch when w0 is
 *             shared ([H,d,d]).
 *   dln_gamma, dln_beta  [H,d] fp32 (out), summed over batch and tokens;
 *             required with LN; without LN NULL, or written with zeros.
 *   workspace  device memory, 256-byte aligned, at least
 *             ttt_linear_backward_workspace_bytes(p) bytes, owned by the
 *             caller; no initialisation needed; scratch after the call; one
 *             call at a time.
 * Outputs and the workspace overlap no input and no other output
 * (TTT_ERR_ALIAS).  Supported: d = 64, mini_batch a positive multiple of
 * 16 (b >= T: batch GD over the whole sequence, the LIT-801 record's item
 * 3), else TTT_ERR_UNSUPPORTED; both io dtypes, any flags.
 * With TTT_BASES_SAVED in p->flags (mini_batch = 16 only, else
 * TTT_ERR_UNSUPPORTED) the workspace must hold the mini-batch bases that
 * ttt_linear_forward_save stored for the same parameters (that flag aside)
 * and inputs; the backward then skips replaying the forward
 * recurrence.  The library cannot check this: stale bases give wrong
 * gradients.
 * gfx950: kernels on hip_stream.  The forward recurrence is replayed (one
 * 512-thread workgroup per unit, unless TTT_BASES_SAVED) and the state at
 * every 16-token tile's start stored in the workspace; the tiles are then
 * walked in reverse.  With mini_batch = 16 the part of every tile that needs
 * no adjoint runs first for all tiles at once (one workgroup per unit and
 * tile, records in the workspace) and the reverse walk (one workgroup per
 * unit) only carries the adjoint; longer mini-batches replay and walk in
 * one launch.  Products at fp32 precision (fp32 matrix-unit products, or
 * exact bf16 products of bf16 inputs with three-part bf16 operands); a last
 * kernel sums dw0 (shared w0), dln_gamma and dln_beta over the batch in a
 * fixed order.  Results are deterministic.
 */
ttt_status ttt_linear_backward(const ttt_params* p,
                               const void* q, const void* k, const void* v,
                               const float* eta, const float* w0,
                               const float* ln_gamma, const float* ln_beta,
                               const void* dz, const float* dw_final,
                               void* dq, void* dk, void* dv, float* deta,
                               float* dw0, float* dln_gamma, float* dln_beta,
                               void* workspace, uint64_t workspace_bytes,
                               void* hip_stream);

/*
 * TTT-MLP forward scan, hidden width `hidden` (m).
 *   w1_0 [H,d,m], b1_0 [H,m], w2_0 [H,m,d], b2_0 [H,d] fp32
 *   (leading B with state0_per_batch).  The biases are state.
 *   w1_out, b1_out, w2_out, b2_out: [B,H,...] fp32, all NULL or all set.
 * Supported: d = 64, hidden = 256, mini_batch = 16, both io dtypes, any
 * flags.
 * gfx950 kernel: one 512-thread workgroup per (batch, head) unit; the state
 * stays in registers across the whole sequence.
 */
ttt_status ttt_mlp_forward(const ttt_params* p, int32_t hidden,
                           const void* q, const void* k, const void* v,
                           const float* eta,
                           const float* w1_0, const float* b1_0,
                           const float* w2_0, const float* b2_0,
                           const float* ln_gamma, const float* ln_beta,
                           void* z, float* w1_out, float* b1_out,
                           float* w2_out, float* b2_out, void* hip_stream);

/*
 * One token of the TTT-MLP scan per (batch, head) unit: the streaming
 * (decode) step, as ttt_linear_decode_step with the state
 * S = (W1, b1, W2, b2).  The gradient is taken at base = (pos == 0 ? S :
 * S_base), S <- S - eta_t * gradient, z_t = f(q_t; S) and, when pos == 0,
 * base is stored into S_base.  Calling it for t = 0, 1, ... with
 * pos = t mod mini_batch, starting from S = S0, reproduces ttt_mlp_forward
 * (the codewithpapers.app record of arXiv 2407.04620, TTT-MLP; the LIT-801
 * record, "Key takeaways" items 1, 2 and 5).
 *   p        T must be 1; mini_batch any b >= 1; state0_per_batch unused.
 *   hidden   m; 256 supported (TTT_ERR_UNSUPPORTED otherwise).
 *   q, k, v  [B,H,d] io_dtype;  eta [B,H] fp32;  z [B,H,d] io_dtype (out).
 *   w1 [B,H,d,m], b1 [B,H,m], w2 [B,H,m,d], b2 [B,H,d] fp32: the state,
 *            read and written in place.
 *   w1_base, b1_base, w2_base, b2_base: the base, same shapes; read when
 *            pos > 0, written when pos == 0.
 * None of the eight state buffers and z overlaps another or an input
 * (TTT_ERR_ALIAS); pos out of range is TTT_ERR_ARG.  gfx950 kernel: one
 * 1024-thread workgroup per unit holding its state in registers, fp32
 * arithmetic; bound by moving the state (about 397 KB per unit and token).
 */
ttt_status ttt_mlp_decode_step(const ttt_params* p, int32_t hidden, int32_t pos,
                               const void* q, const void* k, const void* v,
                               const float* eta,
                               float* w1, float* b1, float* w2, float* b2,
                               float* w1_base, float* b1_base,
                               float* w2_base, float* b2_base,
                               const float* ln_gamma, const float* ln_beta,
                               void* z, void* hip_stream);

/*
 * The TTT-MLP streaming step of ttt_mlp_decode_step with a compact pending
 * state: the same tokens, the same z (up to rounding order).  Within a
 * mini-batch the state after the tokens s < pos is the base plus rank-1
 * terms, W1 = w1_base + sum_s k_s^T u1_s, b1 = b1_base + sum_s u1_s,
 * W2 = w2_base + sum_s a_s^T u2_s, b2 = b2_base + sum_s u2_s, with
 * u1 = -eta * dl/dp, u2 = -eta * dl/do and a = GELU(k W1 + b1), all at the
 * base; the stream carries the base and these rows instead of the state:
 *   w1_base [B,H,d,m], b1_base [B,H,m], w2_base [B,H,m,d], b2_base [B,H,d]
 *           fp32, read; at pos == 0 first replaced by the base plus all
 *           mini_batch history slots (the previous mini-batch).
 *   hist    [B,H,mini_batch,2d+2m] fp32: slot s holds k_s[d], u1_s[m],
 *           a_s[m], u2_s[d]; slot pos is written.  Zero it when a stream
 *           starts.
 * About 165 KB move per unit and token for mini_batch = 16 (397 KB for the
 * (S, S_base) form).  The final state of a ttt_mlp_forward over a whole
 * number of mini-batches starts a stream as the base with a zero history.
 *   p   T must be 1; mini_batch at most 16 (TTT_ERR_UNSUPPORTED).
 * Other arguments, aliasing and errors as ttt_mlp_decode_step.
 */
ttt_status ttt_mlp_decode_step_compact(const ttt_params* p, int32_t hidden, int32_t pos,
                                       const void* q, const void* k, const void* v,
                                       const float* eta,
                                       float* w1_base, float* b1_base,
                                       float* w2_base, float* b2_base, float* hist,
                                       const float* ln_gamma, const float* ln_beta,
                                       void* z, void* hip_stream);

/* Static, NUL-terminated description of a status code. */
const char* ttt_status_string(ttt_status s);

/*
 * Bytes of device workspace that ttt_mlp_backward needs: per unit, the base
 * of every 16-token mini-batch (132,352 bytes each) plus one more state and
 * 180,736 bytes of per-mini-batch intermediates, rounded up to 256 bytes
 * (0 if p fails the common checks or hidden != 256).  About 1.7 GB for
 * B = 8, H = 12, T = 2048.
 */
uint64_t ttt_mlp_backward_workspace_bytes(const ttt_params* p, int32_t hidden);

/*
 * Backward pass of the TTT-MLP forward scan (ttt_mlp_forward: same p,
 * hidden and inputs): the vector-Jacobian product that training needs (the
 * LIT-801 record, "Key takeaways" item 2).  For cotangents dz (and the four
 * d*_final on the final state) it writes the gradients of
 *   L = sum_t <dz_t, z_t> + <dW1_T, W1_T> + <db1_T, b1_T> + <dW2_T, W2_T> + <db2_T, b2_T>
 * with respect to q, k, v, eta, the initial state and gamma, beta.
 *   dz          [B,H,T,d] io_dtype.
 *   d*_final    [B,H,...] fp32 (the final state's shapes), all four or all NULL (zero).
 *   dq, dk, dv  [B,H,T,d] io_dtype (out; rounded once from fp32);  deta [B,H,T] fp32.
 *   dw1, db1, dw2, db2  fp32, the initial state's shapes: [H,...] summed over
 *               the batch, or [B,H,...] with state0_per_batch.
 *   dln_gamma, dln_beta  [H,d] fp32, summed over batch and tokens; required
 *               with LN, may be NULL (both) without it.
 *   workspace   device memory, 256-byte aligned, at least
 *               ttt_mlp_backward_workspace_bytes(p, hidden) bytes, owned by the
 *               caller; no initialisation needed; scratch after the call; one
 *               call at a time.
 * Outputs and the workspace overlap no input and no other output
 * (TTT_ERR_ALIAS).  Supported: d = 64, hidden = 256, mini_batch = 16 (else
 * TTT_ERR_UNSUPPORTED), both io dtypes, any flags.  Products run in fp32 on
 * the matrix unit; the forward recurrence is replayed in the same call.  Two
 * kernels on hip_stream (the scan, then the sums over the batch).
 */
ttt_status ttt_mlp_backward(const ttt_params* p, int32_t hidden,
                            const void* q, const void* k, const void* v,
                            const float* eta,
                            const float* w1_0, const float* b1_0,
                            const float* w2_0, const float* b2_0,
                            const float* ln_gamma, const float* ln_beta,
                            const void* dz,
                            const float* dw1_final, const float* db1_final,
                            const float* dw2_final, const float* db2_final,
                            void* dq, void* dk, void* dv, float* deta,
                            float* dw1, float* db1, float* dw2, float* db2,
                            float* dln_gamma, float* dln_beta,
                            void* workspace, uint64_t workspace_bytes,
                            void* hip_stream);

/*
 * The input side of a TTT layer: q, k, v of every head and the
 * token-dependent learning rate eta, made from the layer input x.  The
 * outer loop trains the projections theta_Q, theta_K, theta_V and a
 * learning rate that depends on the token (the LIT-801 record, "Key
 * takeaways" item 2; the nowfound.app launch page, "In the maker's words",
 * names the QKV projection matrices).  With x [B,T,D] and the stacked
 * weights w_in [3*H*d + H, D] (rows h*d .. h*d + d-1: theta_Q of head h as
 * d rows over D; then theta_K and theta_V the same way; then row
 * 3*H*d + h: the gate of head h):
 *   q[b,h,t,f] = sum_j x[b,t,j] w_in[h*d + f, j]      (k: row H*d + h*d + f,
 *                                                     v: row 2*H*d + h*d + f)
 *   eta[b,h,t] = eta_base / (1 + exp(-(sum_j x[b,t,j] w_in[3*H*d + h, j] + b_eta[h])))
 * The gate's form is a reading: the pages give none; this one is learned,
 * depends on the token and keeps eta in (0, eta_base).
 *   p        B, H, T, d of the scan that consumes the outputs (checked as
 *            for the scan; mini_batch, flags and ln_eps are not used);
 *            io_dtype TTT_BF16 and d = 64, else TTT_ERR_UNSUPPORTED.
 *   d_model  D: a positive multiple of 64 (else TTT_ERR_UNSUPPORTED).
 *   x        [B,T,D] bf16, 16-byte aligned (else TTT_ERR_ARG).
 *   w_in     [3*H*d + H, D] bf16, 16-byte aligned (else TTT_ERR_ARG).
 *   b_eta    [H] fp32.
 *   eta_base finite and > 0 (else TTT_ERR_ARG).
 *   q, k, v  [B,H,T,d] bf16 (out), 16-byte aligned (else TTT_ERR_ARG): the
 *            scan's input layout, each rounded once (to nearest even) from
 *            an fp32 accumulation over D.
 *   eta      [B,H,T] fp32 (out).
 * B*T at most 2^30 (else TTT_ERR_SHAPE).  Outputs overlap no input and no
 * other output (TTT_ERR_ALIAS).
 * gfx950: one kernel on hip_stream: bf16 matrix-unit products (16x16x32,
 * fp32 accumulation), a 256 x 128 output tile per 512-thread workgroup.
 */
ttt_status ttt_input_projection(const ttt_params* p, int32_t d_model,
                                const void* x, const void* w_in,
                                const float* b_eta, float eta_base,
                                void* q, void* k, void* v, float* eta,
                                void* hip_stream);

/* TTT_ABI_VERSION of the built library. */
int32_t ttt_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
