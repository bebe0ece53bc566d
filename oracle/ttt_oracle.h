/*
 * ttt_oracle.h -- plain, slow, fp64 CPU reference of the TTT-layer forward scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU product
 * path shares no code, header, table or helper with it.
 *
 * Sources (web pages about arXiv 2407.04620, "Learning to (Learn at Test
 * Time): RNNs with Expressive Hidden States", Sun et al.):
 *   [KT1..KT6]  dmarx.github.io nucleation literature record LIT-801,
 *               "Key takeaways", items 1..6.
 *   [ABS]       codewithpapers.app paper record, "abstract" field.
 *   [GLOSS]     ai-solutions.wiki glossary "Test-Time Training",
 *               sections "The hidden state as a model" and
 *               "TTT-Linear and TTT-MLP".
 *
 * What is computed (row-vector convention, one independent unit per
 * (batch, head); [KT1]: the state is the weights W of an inner model f,
 * W_t = W_{t-1} - eta_t * grad l(W_{t-1}; x_t), z_t = f(q_t; W_t)):
 *   loss     l(S; k, v) = || f(k; S) - v ||^2            [KT2]
 *   Linear   f(x) = x + LN(x W)                           [ABS], [KT5]
 *   MLP      f(x) = x + LN(GELU(x W1 + b1) W2 + b2)        [ABS], [KT5]
 *   mini-batch inner GD with batch size b [KT5]: every gradient inside a
 *   mini-batch is taken at the state held when the mini-batch began, and
 *   the state absorbs them one token at a time, so z_t sees the updates of
 *   tokens s <= t of its own mini-batch (b = 1 is [KT1]'s online rule,
 *   b = T is [KT3]'s batch GD over the causal prefix).
 *
 * Readings taken where the pages are silent (each is pinned by a test):
 *   - squared Euclidean norm summed over the d outputs, no 1/2, no mean;
 *     gradients of a mini-batch are summed (Theorem 1 in [KT3] fixes the
 *     constant: eta = 1/2 must give coefficient 1);
 *   - eta_t multiplies token t's own gradient, used exactly as given;
 *   - LN over the d features of one token, biased variance, epsilon given
 *     by the caller; gamma/beta are fixed per-head parameters, not state;
 *   - GELU is the exact erf form; the MLP biases b1, b2 are state;
 *   - a last partial mini-batch (T mod b != 0) is one step on its tokens.
 *
 * Layouts: contiguous row-major, d fastest.
 *   q, k, v, z  [B,H,T,d]      eta [B,H,T]
 *   Linear state W  [d,d] (input row index first);
 *   MLP state W1 [d,m], b1 [m], W2 [m,d], b2 [d];
 *   initial state [H,...] shared over the batch, or [B,H,...] when
 *   state0_per_batch != 0.  gamma, beta [H,d].
 * Inputs are fp32 arrays read exactly; all arithmetic and outputs are fp64.
 * Units are independent; threads split units only, so results do not
 * depend on the thread count.  Return value 0 on success, -1 on a bad
 * argument (nothing written), -2 when a thread could not be started.
 */
#ifndef TTT_ORACLE_H
#define TTT_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int B, H, T, d;
  int mini_batch;        /* b >= 1; b >= T means one step per sequence */
  int use_ln;            /* f(x) = [x +] LN(g(x)) when set, [x +] g(x) when 0 */
  int use_residual;      /* add the inner input x to f when set */
  double ln_eps;
  int state0_per_batch;  /* 0: initial state [H,...]; 1: [B,H,...] */
} ttt_oracle_cfg;

int ttt_oracle_linear(const ttt_oracle_cfg* cfg,
                      const float* q, const float* k, const float* v,
                      const float* eta, const float* w0,
                      const float* gamma, const float* beta,
                      double* z, double* w_out, int n_threads);

int ttt_oracle_mlp(const ttt_oracle_cfg* cfg, int hidden,
                   const float* q, const float* k, const float* v,
                   const float* eta,
                   const float* w1_0, const float* b1_0,
                   const float* w2_0, const float* b2_0,
                   const float* gamma, const float* beta,
                   double* z, double* w1_out, double* b1_out,
                   double* w2_out, double* b2_out, int n_threads);

/* One token's loss l(W; k, v) and, when gW is not NULL, its gradient with
 * respect to W ([d,d]).  gamma/beta are read only when use_ln is set. */
double ttt_oracle_linear_loss_grad(int d, int use_ln, int use_residual,
                                   double ln_eps, const double* W,
                                   const double* k, const double* v,
                                   const double* gamma, const double* beta,
                                   double* gW);

/* Same for the MLP state (W1 [d,m], b1 [m], W2 [m,d], b2 [d]).  The four
 * gradient pointers are either all NULL or all valid. */
double ttt_oracle_mlp_loss_grad(int d, int m, int use_ln, int use_residual,
                                double ln_eps,
                                const double* W1, const double* b1,
                                const double* W2, const double* b2,
                                const double* k, const double* v,
                                const double* gamma, const double* beta,
                                double* gW1, double* gb1,
                                double* gW2, double* gb2);

/* Inner-model forward f(x; S) for one token (the output rule of [KT1]). */
void ttt_oracle_linear_apply(int d, int use_ln, int use_residual,
                             double ln_eps, const double* W, const double* x,
                             const double* gamma, const double* beta,
                             double* out);
void ttt_oracle_mlp_apply(int d, int m, int use_ln, int use_residual,
                          double ln_eps, const double* W1, const double* b1,
                          const double* W2, const double* b2, const double* x,
                          const double* gamma, const double* beta,
                          double* out);

#ifdef __cplusplus
}
#endif
#endif
