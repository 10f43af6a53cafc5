/*
 * ttt_oracle.c -- slow, plain fp64 CPU oracle for the TTT-layer forward pass and
 * the backward of TTT-Linear.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file. Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it. It shares no source, header, table or helper with the HIP library.
 *
 * What it computes (every quantity in fp64, loops written out, no blocking):
 *
 *   Inner model f and per-token self-supervised loss
 *     l_t(theta) = || f(k_t; theta) - v_t ||^2
 *   Web page "Test-Time Training: Linear Complexity Beyond Attention",
 *   section "1. The Self-Supervised Inner-Loop Task", writes the loss as
 *   (1/2)||W k - v||^2 with f(k;W) = W k. Here f acts on row vectors,
 *   f(x;W) = x W, and the loss carries no 1/2; that is the same method with
 *   W_page = W^T and eta_page = 2 eta (a test checks the equivalence).
 *
 *   Inner models:
 *     PLAIN : f(x;W) = x W                                   (page 1, sec. 1)
 *     LN    : f(x;W) = x + LN(x W)
 *             page 1 sec. 3 applies LayerNorm plus a residual to the layer
 *             output; this variant places them inside the inner model.
 *     MLP   : f(x;W1,W2) = x + LN(GELU(x W1) W2)
 *             page "How to Master Test-Time Training for Infinite Context
 *             LLMs", section "The Math and Architecture of TTT Layers", names
 *             a small multi-layer perceptron as the inner model. GELU is the
 *             exact erf form; there are no biases.
 *     LN(h) = gamma * (h - mean(h)) / sqrt(var(h) + eps) + beta over the last
 *     axis, biased variance, gamma/beta fixed (not updated by the inner step).
 *
 *   Three ways of running the inner loop over a sequence (mode):
 *     ONLINE    token-by-token gradient descent, page 1 section "2. The Online
 *               Gradient Descent Update Rule":
 *                 theta <- theta - eta_t grad l_t(theta);  z_t = f(q_t; theta)
 *               (section "3. Forward Evaluation": the output uses the weights
 *               already updated with token t).
 *     MINIBATCH mini-batch primal form, page 1 section "4. Mini-Batch
 *               Parallelism (Dual Formulation)": tokens are grouped into
 *               mini-batches of b; every gradient inside a mini-batch is taken
 *               at the mini-batch's starting weights theta_c, and the per-token
 *               weights theta_t = theta_c - sum_{s<=t in batch} eta_s grad l_s(theta_c)
 *               are materialised explicitly to evaluate z_t = f(q_t; theta_t).
 *               This is the result of record.
 *     DUAL      the same mini-batch computation written with matrices, the
 *               form that section says mirrors causal attention:
 *                 G   = d l / d(pre-activation) at theta_c (rows = tokens)
 *                 Z   = f evaluated on  Q W_c - tril(Q K^T) diag(eta) G
 *                 W  <- W_c - K^T diag(eta) G
 *               tril includes the diagonal. The MLP applies this to each layer.
 *     BLOCK_BEFORE, BLOCK_AFTER
 *               block-causal large chunks. Page "Test-Time Training Done Right"
 *               (abstract) argues for large mini-batches and contrasts them with
 *               the fine-grained block-wise causal dependencies of small ones;
 *               read plainly, a large chunk takes one step with every gradient
 *               at its starting weights (as MINIBATCH) and its tokens' outputs
 *               use one set of weights for the whole chunk, with no causal
 *               mask inside it: the weights before the chunk's step
 *               (BLOCK_BEFORE: z_t = f(q_t; theta_c)) or after it (BLOCK_AFTER:
 *               z_t = f(q_t; theta_{c+1})). The state sequence, and so the final
 *               state, equals MINIBATCH's.
 *
 * Layouts (row-major, C order): Q,K,V [B,H,N,d]; eta [B,H,N]; W0 [B,H,d,d]
 * (row index = input feature); W1 [B,H,d,hid]; W2 [B,H,hid,d]; gamma, beta
 * [H,d]; Z [B,H,N,d]. The last mini-batch holds N mod b tokens when b does not
 * divide N. Units (b,h) are independent and run in an OpenMP loop.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define MODE_ONLINE 0
#define MODE_MINIBATCH 1
#define MODE_DUAL 2
#define MODE_BLOCK_BEFORE 3
#define MODE_BLOCK_AFTER 4
#define KIND_PLAIN 0
#define KIND_LN 1

/* ------------------------------------------------------------------------ */
/* small dense helpers, fp64                                                 */
/* ------------------------------------------------------------------------ */

/* y[n] = sum_i x[i] * M[i][n],  M is [m x n] row-major */
static void vec_mat(int m, int n, const double* x, const double* M, double* y)
{
    for (int j = 0; j < n; ++j) {
        double s = 0.0;
        for (int i = 0; i < m; ++i) s += x[i] * M[(size_t)i * n + j];
        y[j] = s;
    }
}

/* y[i] = sum_n M[i][n] * x[n] */
static void mat_vec(int m, int n, const double* M, const double* x, double* y)
{
    for (int i = 0; i < m; ++i) {
        double s = 0.0;
        for (int j = 0; j < n; ++j) s += M[(size_t)i * n + j] * x[j];
        y[i] = s;
    }
}

static double dot(int n, const double* a, const double* b)
{
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

/* M[i][j] -= alpha * a[i] * g[j]  (rank-one gradient step, M is [m x n]) */
static void rank1_sub(int m, int n, double alpha, const double* a, const double* g, double* M)
{
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < n; ++j) M[(size_t)i * n + j] -= alpha * a[i] * g[j];
}

/* ------------------------------------------------------------------------ */
/* LayerNorm and GELU, forward and backward                                  */
/* ------------------------------------------------------------------------ */

/* Forward: xhat = (h - mu) * r, y = gamma*xhat + beta; returns r. */
static double ln_forward(int d, const double* h, const double* gamma, const double* beta,
                         double eps, double* xhat, double* y)
{
    double mu = 0.0;
    for (int j = 0; j < d; ++j) mu += h[j];
    mu /= d;
    double var = 0.0;
    for (int j = 0; j < d; ++j) var += (h[j] - mu) * (h[j] - mu);
    var /= d;
    double r = 1.0 / sqrt(var + eps);
    for (int j = 0; j < d; ++j) {
        xhat[j] = (h[j] - mu) * r;
        y[j] = gamma[j] * xhat[j] + beta[j];
    }
    return r;
}

/* Backward of y = LN(h) given dy: dh = r*(dxh - mean(dxh) - xhat*mean(dxh*xhat)),
 * dxh = dy*gamma. */
static void ln_backward(int d, const double* xhat, double r, const double* gamma,
                        const double* dy, double* dh)
{
    double m1 = 0.0, m2 = 0.0;
    for (int j = 0; j < d; ++j) {
        double dxh = dy[j] * gamma[j];
        m1 += dxh;
        m2 += dxh * xhat[j];
    }
    m1 /= d;
    m2 /= d;
    for (int j = 0; j < d; ++j) {
        double dxh = dy[j] * gamma[j];
        dh[j] = r * (dxh - m1 - xhat[j] * m2);
    }
}

static double gelu(double a) { return 0.5 * a * (1.0 + erf(a / sqrt(2.0))); }

/* d/da [a * Phi(a)] = Phi(a) + a * phi(a) */
static double gelu_prime(double a)
{
    const double inv_sqrt_2pi = 0.39894228040143267794;
    return 0.5 * (1.0 + erf(a / sqrt(2.0))) + a * inv_sqrt_2pi * exp(-0.5 * a * a);
}

/* ------------------------------------------------------------------------ */
/* Linear inner model (PLAIN or LN)                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
    int kind, d;
    const double *gamma, *beta;
    double eps;
} lin_model;

/* out = f(x; W). scratch needs 2*d doubles. */
static void lin_f(const lin_model* m, const double* W, const double* x, double* out, double* scratch)
{
    int d = m->d;
    if (m->kind == KIND_PLAIN) {
        vec_mat(d, d, x, W, out);
        return;
    }
    double* h = scratch;
    double* xh = scratch + d;
    vec_mat(d, d, x, W, h);
    ln_forward(d, h, m->gamma, m->beta, m->eps, xh, out);
    for (int j = 0; j < d; ++j) out[j] += x[j];
}

/* g = d l / d h for l = ||f(k;W) - v||^2, where h = k W is the pre-activation.
 * The weight gradient is then k^T g. scratch needs 4*d doubles. */
static void lin_preact_grad(const lin_model* m, const double* W, const double* k, const double* v,
                            double* g, double* scratch)
{
    int d = m->d;
    double* h = scratch;
    double* xh = scratch + d;
    double* y = scratch + 2 * d;
    double* dy = scratch + 3 * d;
    vec_mat(d, d, k, W, h);
    if (m->kind == KIND_PLAIN) {
        for (int j = 0; j < d; ++j) g[j] = 2.0 * (h[j] - v[j]);
        return;
    }
    double r = ln_forward(d, h, m->gamma, m->beta, m->eps, xh, y);
    for (int j = 0; j < d; ++j) dy[j] = 2.0 * (k[j] + y[j] - v[j]);
    ln_backward(d, xh, r, m->gamma, dy, g);
}

static double lin_loss(const lin_model* m, const double* W, const double* k, const double* v,
                       double* scratch)
{
    int d = m->d;
    double* f = scratch + 2 * d;
    lin_f(m, W, k, f, scratch);
    double s = 0.0;
    for (int j = 0; j < d; ++j) s += (f[j] - v[j]) * (f[j] - v[j]);
    return s;
}

/* One (sequence, head) unit. */
static void lin_unit(int mode, const lin_model* m, int N, int b, const double* Q, const double* K,
                     const double* V, const double* eta, const double* W0, double* Z, double* Wend)
{
    int d = m->d;
    size_t dd = (size_t)d * d;
    double* W = malloc(dd * sizeof(double));   /* running state */
    double* Wc = malloc(dd * sizeof(double));  /* mini-batch starting weights */
    double* scratch = malloc(4 * (size_t)d * sizeof(double));
    double* g = malloc((size_t)d * sizeof(double));
    memcpy(W, W0, dd * sizeof(double));

    if (mode == MODE_ONLINE) {
        for (int t = 0; t < N; ++t) {
            lin_preact_grad(m, W, K + (size_t)t * d, V + (size_t)t * d, g, scratch);
            rank1_sub(d, d, eta[t], K + (size_t)t * d, g, W);
            lin_f(m, W, Q + (size_t)t * d, Z + (size_t)t * d, scratch);
        }
    } else if (mode == MODE_MINIBATCH) {
        for (int c0 = 0; c0 < N; c0 += b) {
            int c1 = c0 + b < N ? c0 + b : N;
            memcpy(Wc, W, dd * sizeof(double));
            for (int t = c0; t < c1; ++t) {
                lin_preact_grad(m, Wc, K + (size_t)t * d, V + (size_t)t * d, g, scratch);
                rank1_sub(d, d, eta[t], K + (size_t)t * d, g, W);
                lin_f(m, W, Q + (size_t)t * d, Z + (size_t)t * d, scratch);
            }
        }
    } else if (mode == MODE_BLOCK_BEFORE || mode == MODE_BLOCK_AFTER) {
        for (int c0 = 0; c0 < N; c0 += b) {
            int c1 = c0 + b < N ? c0 + b : N;
            memcpy(Wc, W, dd * sizeof(double));
            /* one step for the whole chunk, every gradient at theta_c */
            for (int t = c0; t < c1; ++t) {
                lin_preact_grad(m, Wc, K + (size_t)t * d, V + (size_t)t * d, g, scratch);
                rank1_sub(d, d, eta[t], K + (size_t)t * d, g, W);
            }
            const double* Wout = mode == MODE_BLOCK_BEFORE ? Wc : W;
            for (int t = c0; t < c1; ++t) lin_f(m, Wout, Q + (size_t)t * d, Z + (size_t)t * d, scratch);
        }
    } else { /* MODE_DUAL */
        double* G = malloc((size_t)b * d * sizeof(double));
        double* hq = malloc((size_t)d * sizeof(double));
        double* xh = malloc((size_t)d * sizeof(double));
        for (int c0 = 0; c0 < N; c0 += b) {
            int c1 = c0 + b < N ? c0 + b : N;
            int n = c1 - c0;
            const double* Qc = Q + (size_t)c0 * d;
            const double* Kc = K + (size_t)c0 * d;
            const double* Vc = V + (size_t)c0 * d;
            /* G: pre-activation gradients of every token in the batch at W_c */
            for (int s = 0; s < n; ++s)
                lin_preact_grad(m, W, Kc + (size_t)s * d, Vc + (size_t)s * d, G + (size_t)s * d, scratch);
            /* H_Q = Q W_c - tril(Q K^T) diag(eta) G */
            for (int t = 0; t < n; ++t) {
                vec_mat(d, d, Qc + (size_t)t * d, W, hq);
                for (int s = 0; s <= t; ++s) {
                    double a = dot(d, Qc + (size_t)t * d, Kc + (size_t)s * d) * eta[c0 + s];
                    for (int j = 0; j < d; ++j) hq[j] -= a * G[(size_t)s * d + j];
                }
                double* z = Z + (size_t)(c0 + t) * d;
                if (m->kind == KIND_PLAIN) {
                    memcpy(z, hq, (size_t)d * sizeof(double));
                } else {
                    ln_forward(d, hq, m->gamma, m->beta, m->eps, xh, z);
                    for (int j = 0; j < d; ++j) z[j] += Qc[(size_t)t * d + j];
                }
            }
            /* W <- W_c - K^T diag(eta) G */
            for (int s = 0; s < n; ++s)
                rank1_sub(d, d, eta[c0 + s], Kc + (size_t)s * d, G + (size_t)s * d, W);
        }
        free(G);
        free(hq);
        free(xh);
    }
    memcpy(Wend, W, dd * sizeof(double));
    free(W);
    free(Wc);
    free(scratch);
    free(g);
}

/* Returns 0 on success, -1 on a bad argument. */
int ttt_oracle_linear(int mode, int kind, int B, int H, int N, int d, int b, const double* Q,
                      const double* K, const double* V, const double* eta, const double* W0,
                      const double* gamma, const double* beta, double eps, double* Z, double* Wend,
                      int nthreads)
{
    if (mode < 0 || mode > 4 || (kind != KIND_PLAIN && kind != KIND_LN)) return -1;
    if (B < 1 || H < 1 || N < 0 || d < 1 || b < 1) return -1;
    if (kind == KIND_LN && (!gamma || !beta)) return -1;
    int units = B * H;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int u = 0; u < units; ++u) {
        int h = u % H;
        lin_model m = {kind, d, kind == KIND_LN ? gamma + (size_t)h * d : NULL,
                       kind == KIND_LN ? beta + (size_t)h * d : NULL, eps};
        size_t so = (size_t)u * N * d;
        lin_unit(mode, &m, N, b, Q + so, K + so, V + so, eta + (size_t)u * N, W0 + (size_t)u * d * d,
                 Z + so, Wend + (size_t)u * d * d);
    }
    return 0;
}

double ttt_oracle_linear_loss(int kind, int d, const double* W, const double* k, const double* v,
                              const double* gamma, const double* beta, double eps)
{
    lin_model m = {kind, d, gamma, beta, eps};
    double* scratch = malloc(4 * (size_t)d * sizeof(double));
    double l = lin_loss(&m, W, k, v, scratch);
    free(scratch);
    return l;
}

/* dW[i][j] = d l / d W[i][j] = k[i] * g[j] */
void ttt_oracle_linear_grad(int kind, int d, const double* W, const double* k, const double* v,
                            const double* gamma, const double* beta, double eps, double* dW)
{
    lin_model m = {kind, d, gamma, beta, eps};
    double* scratch = malloc(4 * (size_t)d * sizeof(double));
    double* g = malloc((size_t)d * sizeof(double));
    lin_preact_grad(&m, W, k, v, g, scratch);
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) dW[(size_t)i * d + j] = k[i] * g[j];
    free(scratch);
    free(g);
}

/* ------------------------------------------------------------------------ */
/* MLP inner model: f(x) = x + LN(GELU(x W1) W2)                             */
/* ------------------------------------------------------------------------ */

typedef struct {
    int d, hid;
    const double *gamma, *beta;
    double eps;
} mlp_model;

typedef struct {
    double *a, *x2, *h, *xh, *y, *dy, *g2, *g1;
} mlp_scratch;

static void mlp_scratch_alloc(const mlp_model* m, mlp_scratch* s)
{
    s->a = malloc((size_t)m->hid * sizeof(double));
    s->x2 = malloc((size_t)m->hid * sizeof(double));
    s->g1 = malloc((size_t)m->hid * sizeof(double));
    s->h = malloc((size_t)m->d * sizeof(double));
    s->xh = malloc((size_t)m->d * sizeof(double));
    s->y = malloc((size_t)m->d * sizeof(double));
    s->dy = malloc((size_t)m->d * sizeof(double));
    s->g2 = malloc((size_t)m->d * sizeof(double));
}

static void mlp_scratch_free(mlp_scratch* s)
{
    free(s->a); free(s->x2); free(s->g1); free(s->h);
    free(s->xh); free(s->y); free(s->dy); free(s->g2);
}

static void mlp_f(const mlp_model* m, const double* W1, const double* W2, const double* x,
                  double* out, mlp_scratch* s)
{
    vec_mat(m->d, m->hid, x, W1, s->a);
    for (int j = 0; j < m->hid; ++j) s->x2[j] = gelu(s->a[j]);
    vec_mat(m->hid, m->d, s->x2, W2, s->h);
    ln_forward(m->d, s->h, m->gamma, m->beta, m->eps, s->xh, out);
    for (int j = 0; j < m->d; ++j) out[j] += x[j];
}

/* Fills s->a (= k W1), s->x2 (= GELU(a)), s->g2 (= dl/dh, h = x2 W2) and
 * s->g1 (= dl/da). Weight gradients: dW1 = k^T g1, dW2 = x2^T g2. */
static void mlp_grads(const mlp_model* m, const double* W1, const double* W2, const double* k,
                      const double* v, mlp_scratch* s)
{
    int d = m->d, hid = m->hid;
    vec_mat(d, hid, k, W1, s->a);
    for (int j = 0; j < hid; ++j) s->x2[j] = gelu(s->a[j]);
    vec_mat(hid, d, s->x2, W2, s->h);
    double r = ln_forward(d, s->h, m->gamma, m->beta, m->eps, s->xh, s->y);
    for (int j = 0; j < d; ++j) s->dy[j] = 2.0 * (k[j] + s->y[j] - v[j]);
    ln_backward(d, s->xh, r, m->gamma, s->dy, s->g2);
    mat_vec(hid, d, W2, s->g2, s->g1); /* g2 W2^T */
    for (int j = 0; j < hid; ++j) s->g1[j] *= gelu_prime(s->a[j]);
}

static void mlp_unit(int mode, const mlp_model* m, int N, int b, const double* Q, const double* K,
                     const double* V, const double* eta, const double* W1_0, const double* W2_0,
                     double* Z, double* W1e, double* W2e)
{
    int d = m->d, hid = m->hid;
    size_t n1 = (size_t)d * hid;
    double* W1 = malloc(n1 * sizeof(double));
    double* W2 = malloc(n1 * sizeof(double));
    double* W1c = malloc(n1 * sizeof(double));
    double* W2c = malloc(n1 * sizeof(double));
    mlp_scratch s;
    mlp_scratch_alloc(m, &s);
    memcpy(W1, W1_0, n1 * sizeof(double));
    memcpy(W2, W2_0, n1 * sizeof(double));

    if (mode == MODE_ONLINE) {
        for (int t = 0; t < N; ++t) {
            mlp_grads(m, W1, W2, K + (size_t)t * d, V + (size_t)t * d, &s);
            rank1_sub(d, hid, eta[t], K + (size_t)t * d, s.g1, W1);
            rank1_sub(hid, d, eta[t], s.x2, s.g2, W2);
            mlp_f(m, W1, W2, Q + (size_t)t * d, Z + (size_t)t * d, &s);
        }
    } else if (mode == MODE_MINIBATCH) {
        for (int c0 = 0; c0 < N; c0 += b) {
            int c1 = c0 + b < N ? c0 + b : N;
            memcpy(W1c, W1, n1 * sizeof(double));
            memcpy(W2c, W2, n1 * sizeof(double));
            for (int t = c0; t < c1; ++t) {
                mlp_grads(m, W1c, W2c, K + (size_t)t * d, V + (size_t)t * d, &s);
                rank1_sub(d, hid, eta[t], K + (size_t)t * d, s.g1, W1);
                rank1_sub(hid, d, eta[t], s.x2, s.g2, W2);
                mlp_f(m, W1, W2, Q + (size_t)t * d, Z + (size_t)t * d, &s);
            }
        }
    } else { /* MODE_DUAL */
        double* G1 = malloc((size_t)b * hid * sizeof(double));
        double* G2 = malloc((size_t)b * d * sizeof(double));
        double* X2 = malloc((size_t)b * hid * sizeof(double));
        double* aq = malloc((size_t)hid * sizeof(double));
        double* x2q = malloc((size_t)hid * sizeof(double));
        double* hq = malloc((size_t)d * sizeof(double));
        double* xh = malloc((size_t)d * sizeof(double));
        for (int c0 = 0; c0 < N; c0 += b) {
            int c1 = c0 + b < N ? c0 + b : N;
            int n = c1 - c0;
            const double* Qc = Q + (size_t)c0 * d;
            const double* Kc = K + (size_t)c0 * d;
            const double* Vc = V + (size_t)c0 * d;
            for (int r = 0; r < n; ++r) {
                mlp_grads(m, W1, W2, Kc + (size_t)r * d, Vc + (size_t)r * d, &s);
                memcpy(G1 + (size_t)r * hid, s.g1, (size_t)hid * sizeof(double));
                memcpy(G2 + (size_t)r * d, s.g2, (size_t)d * sizeof(double));
                memcpy(X2 + (size_t)r * hid, s.x2, (size_t)hid * sizeof(double));
            }
            for (int t = 0; t < n; ++t) {
                const double* q = Qc + (size_t)t * d;
                /* first layer: A_Q = Q W1_c - tril(Q K^T) diag(eta) G1 */
                vec_mat(d, hid, q, W1, aq);
                for (int r = 0; r <= t; ++r) {
                    double a = dot(d, q, Kc + (size_t)r * d) * eta[c0 + r];
                    for (int j = 0; j < hid; ++j) aq[j] -= a * G1[(size_t)r * hid + j];
                }
                for (int j = 0; j < hid; ++j) x2q[j] = gelu(aq[j]);
                /* second layer: H_Q = X2_Q W2_c - tril(X2_Q X2^T) diag(eta) G2 */
                vec_mat(hid, d, x2q, W2, hq);
                for (int r = 0; r <= t; ++r) {
                    double a = dot(hid, x2q, X2 + (size_t)r * hid) * eta[c0 + r];
                    for (int j = 0; j < d; ++j) hq[j] -= a * G2[(size_t)r * d + j];
                }
                double* z = Z + (size_t)(c0 + t) * d;
                ln_forward(d, hq, m->gamma, m->beta, m->eps, xh, z);
                for (int j = 0; j < d; ++j) z[j] += q[j];
            }
            for (int r = 0; r < n; ++r) {
                rank1_sub(d, hid, eta[c0 + r], Kc + (size_t)r * d, G1 + (size_t)r * hid, W1);
                rank1_sub(hid, d, eta[c0 + r], X2 + (size_t)r * hid, G2 + (size_t)r * d, W2);
            }
        }
        free(G1); free(G2); free(X2); free(aq); free(x2q); free(hq); free(xh);
    }
    memcpy(W1e, W1, n1 * sizeof(double));
    memcpy(W2e, W2, n1 * sizeof(double));
    free(W1); free(W2); free(W1c); free(W2c);
    mlp_scratch_free(&s);
}

int ttt_oracle_mlp(int mode, int B, int H, int N, int d, int hid, int b, const double* Q,
                   const double* K, const double* V, const double* eta, const double* W1_0,
                   const double* W2_0, const double* gamma, const double* beta, double eps,
                   double* Z, double* W1e, double* W2e, int nthreads)
{
    if (mode < 0 || mode > 2) return -1;
    if (B < 1 || H < 1 || N < 0 || d < 1 || hid < 1 || b < 1 || !gamma || !beta) return -1;
    int units = B * H;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int u = 0; u < units; ++u) {
        int h = u % H;
        mlp_model m = {d, hid, gamma + (size_t)h * d, beta + (size_t)h * d, eps};
        size_t so = (size_t)u * N * d;
        size_t wo = (size_t)u * d * hid;
        mlp_unit(mode, &m, N, b, Q + so, K + so, V + so, eta + (size_t)u * N, W1_0 + wo, W2_0 + wo,
                 Z + so, W1e + wo, W2e + wo);
    }
    return 0;
}

double ttt_oracle_mlp_loss(int d, int hid, const double* W1, const double* W2, const double* k,
                           const double* v, const double* gamma, const double* beta, double eps)
{
    mlp_model m = {d, hid, gamma, beta, eps};
    mlp_scratch s;
    mlp_scratch_alloc(&m, &s);
    double* f = malloc((size_t)d * sizeof(double));
    mlp_f(&m, W1, W2, k, f, &s);
    double l = 0.0;
    for (int j = 0; j < d; ++j) l += (f[j] - v[j]) * (f[j] - v[j]);
    free(f);
    mlp_scratch_free(&s);
    return l;
}

void ttt_oracle_mlp_grad(int d, int hid, const double* W1, const double* W2, const double* k,
                         const double* v, const double* gamma, const double* beta, double eps,
                         double* dW1, double* dW2)
{
    mlp_model m = {d, hid, gamma, beta, eps};
    mlp_scratch s;
    mlp_scratch_alloc(&m, &s);
    mlp_grads(&m, W1, W2, k, v, &s);
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < hid; ++j) dW1[(size_t)i * hid + j] = k[i] * s.g1[j];
    for (int i = 0; i < hid; ++i)
        for (int j = 0; j < d; ++j) dW2[(size_t)i * d + j] = s.x2[i] * s.g2[j];
    mlp_scratch_free(&s);
}

/* Scalar helpers exposed so tests can pin them against closed forms. */
double ttt_oracle_gelu(double a) { return gelu(a); }
double ttt_oracle_gelu_prime(double a) { return gelu_prime(a); }

/* ------------------------------------------------------------------------ */
/* Backward of TTT-Linear (PLAIN or LN) through the mini-batch dual form     */
/* ------------------------------------------------------------------------ */
/*
 * Reverse-mode differentiation of the DUAL computation above (its result is
 * MINIBATCH's), for outer-loop training: page 1 section "1. The
 * Self-Supervised Inner-Loop Task" has the projections and layer norms trained
 * by ordinary backpropagation through the inner loop. Given the gradients of a
 * scalar objective with respect to the outputs, dZ [B,H,N,d] and dW_end
 * [B,H,d,d], it returns the gradients with respect to every input: dQ, dK, dV
 * [B,H,N,d], deta [B,H,N], dW0 [B,H,d,d] and, for LN, dgamma and dbeta [H,d]
 * summed over the batch. The chunk-start weights W_c are recomputed by a
 * forward pass and kept; the chunks are then visited in reverse with the
 * weight gradient carried from chunk c+1 to chunk c. Per chunk, in the
 * notation of the forward (row vectors, a_ts = q_t . k_s, s <= t):
 *   h_s = k_s W_c,  g_s = d l_s / d h_s,
 *   hq_t = q_t W_c - sum_{s<=t} a_ts eta_s g_s,  z_t = hq_t or q_t + LN(hq_t),
 *   W_{c+1} = W_c - sum_s eta_s k_s^T g_s.
 */

/* Backward of g = d l / d h (lin_preact_grad) given dg. Adds k^T dh to dW and the
 * contributions to dk, dv, dgamma, dbeta. scratch needs 8*d doubles. */
static void lin_preact_grad_bwd(const lin_model* m, const double* W, const double* k, const double* v,
                                const double* dg, double* dW, double* dk, double* dv, double* dgam,
                                double* dbet, double* scratch)
{
    int d = m->d;
    double* h = scratch;
    double* dh = scratch + d;
    vec_mat(d, d, k, W, h);
    if (m->kind == KIND_PLAIN) {
        /* g = 2 (h - v) */
        for (int j = 0; j < d; ++j) {
            dh[j] = 2.0 * dg[j];
            dv[j] -= 2.0 * dg[j];
        }
    } else {
        /* g = r (gx - m1 - xhat m2), gx = gamma dy, dy = 2 (k + gamma xhat + beta - v),
         * xhat = c r, c = h - mu, r = (var + eps)^(-1/2), var = mean(c^2),
         * m1 = mean(gx), m2 = mean(gx xhat). */
        const double* gam = m->gamma;
        const double* bet = m->beta;
        double* c = scratch + 2 * d;
        double* xh = scratch + 3 * d;
        double* dy = scratch + 4 * d;
        double* gx = scratch + 5 * d;
        double* dxh = scratch + 6 * d;
        double* dgx = scratch + 7 * d;
        double mu = 0.0;
        for (int j = 0; j < d; ++j) mu += h[j];
        mu /= d;
        double var = 0.0;
        for (int j = 0; j < d; ++j) {
            c[j] = h[j] - mu;
            var += c[j] * c[j];
        }
        var /= d;
        double r = 1.0 / sqrt(var + m->eps);
        double m1 = 0.0, m2 = 0.0;
        for (int j = 0; j < d; ++j) {
            xh[j] = c[j] * r;
            dy[j] = 2.0 * (k[j] + gam[j] * xh[j] + bet[j] - v[j]);
            gx[j] = gam[j] * dy[j];
            m1 += gx[j];
            m2 += gx[j] * xh[j];
        }
        m1 /= d;
        m2 /= d;
        /* through g = r (gx - m1 - xhat m2) */
        double dr = 0.0, s1 = 0.0, s2 = 0.0;
        for (int j = 0; j < d; ++j) {
            dr += dg[j] * (gx[j] - m1 - xh[j] * m2);
            s1 += dg[j];
            s2 += dg[j] * xh[j];
        }
        double dm1 = -r * s1, dm2 = -r * s2;
        for (int j = 0; j < d; ++j) {
            dgx[j] = r * dg[j] + dm1 / d + dm2 * xh[j] / d;
            dxh[j] = -r * dg[j] * m2 + dm2 * gx[j] / d;
        }
        /* through gx = gamma dy and dy = 2 (k + gamma xhat + beta - v) */
        for (int j = 0; j < d; ++j) {
            dgam[j] += dgx[j] * dy[j];
            double ddy = dgx[j] * gam[j];
            dk[j] += 2.0 * ddy;
            dgam[j] += 2.0 * ddy * xh[j];
            dxh[j] += 2.0 * ddy * gam[j];
            dbet[j] += 2.0 * ddy;
            dv[j] -= 2.0 * ddy;
        }
        /* through xhat = c r, r = (var + eps)^(-1/2), var = mean(c^2), c = h - mu */
        for (int j = 0; j < d; ++j) dr += dxh[j] * c[j];
        double dvar = -0.5 * dr * r * r * r;
        double mean_dc = 0.0;
        for (int j = 0; j < d; ++j) {
            dh[j] = dxh[j] * r + dvar * 2.0 * c[j] / d;   /* dc for now */
            mean_dc += dh[j];
        }
        mean_dc /= d;
        for (int j = 0; j < d; ++j) dh[j] -= mean_dc;
    }
    /* h = k W */
    for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int j = 0; j < d; ++j) {
            acc += dh[j] * W[(size_t)i * d + j];
            dW[(size_t)i * d + j] += k[i] * dh[j];
        }
        dk[i] += acc;
    }
}

/* One (sequence, head) unit. dgam, dbet are per-unit partial sums. */
static void lin_unit_bwd(const lin_model* m, int N, int b, const double* Q, const double* K, const double* V,
                         const double* eta, const double* W0, const double* dZ, const double* dWend,
                         double* dQ, double* dK, double* dV, double* deta, double* dW0, double* dgam,
                         double* dbet)
{
    int d = m->d;
    size_t dd = (size_t)d * d;
    int C = (N + b - 1) / b;
    double* Ws = malloc((size_t)(C > 0 ? C : 1) * dd * sizeof(double));  /* W_c of every chunk */
    double* W = malloc(dd * sizeof(double));
    double* dW = malloc(dd * sizeof(double));
    double* G = malloc((size_t)b * d * sizeof(double));
    double* dG = malloc((size_t)b * d * sizeof(double));
    double* hq = malloc((size_t)d * sizeof(double));
    double* dhq = malloc((size_t)d * sizeof(double));
    double* xh = malloc((size_t)d * sizeof(double));
    double* y = malloc((size_t)d * sizeof(double));
    double* kd = malloc((size_t)d * sizeof(double));
    double* scratch = malloc(8 * (size_t)d * sizeof(double));

    /* forward: the chunk-start weights */
    memcpy(W, W0, dd * sizeof(double));
    for (int c = 0; c < C; ++c) {
        int c0 = c * b, n = (c0 + b < N ? c0 + b : N) - c0;
        memcpy(Ws + (size_t)c * dd, W, dd * sizeof(double));
        for (int s = 0; s < n; ++s)
            lin_preact_grad(m, Ws + (size_t)c * dd, K + (size_t)(c0 + s) * d, V + (size_t)(c0 + s) * d,
                            G + (size_t)s * d, scratch);
        for (int s = 0; s < n; ++s)
            rank1_sub(d, d, eta[c0 + s], K + (size_t)(c0 + s) * d, G + (size_t)s * d, W);
    }

    memset(dQ, 0, (size_t)N * d * sizeof(double));
    memset(dK, 0, (size_t)N * d * sizeof(double));
    memset(dV, 0, (size_t)N * d * sizeof(double));
    memset(deta, 0, (size_t)N * sizeof(double));
    if (dWend) memcpy(dW, dWend, dd * sizeof(double));
    else memset(dW, 0, dd * sizeof(double));

    for (int c = C - 1; c >= 0; --c) {
        int c0 = c * b, n = (c0 + b < N ? c0 + b : N) - c0;
        const double* Wc = Ws + (size_t)c * dd;
        const double* Qc = Q + (size_t)c0 * d;
        const double* Kc = K + (size_t)c0 * d;
        const double* Vc = V + (size_t)c0 * d;
        const double* et = eta + c0;
        double* dQc = dQ + (size_t)c0 * d;
        double* dKc = dK + (size_t)c0 * d;
        double* dVc = dV + (size_t)c0 * d;
        double* dec = deta + c0;
        for (int s = 0; s < n; ++s)
            lin_preact_grad(m, Wc, Kc + (size_t)s * d, Vc + (size_t)s * d, G + (size_t)s * d, scratch);
        memset(dG, 0, (size_t)n * d * sizeof(double));

        /* W_{c+1} = W_c - sum_s eta_s k_s^T g_s, with dW holding d/dW_{c+1} */
        for (int s = 0; s < n; ++s) {
            const double* ks = Kc + (size_t)s * d;
            const double* gs = G + (size_t)s * d;
            vec_mat(d, d, ks, dW, kd);                       /* k_s dW */
            double kdg = dot(d, kd, gs);                      /* k_s dW g_s^T */
            for (int j = 0; j < d; ++j) dG[(size_t)s * d + j] -= et[s] * kd[j];
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int j = 0; j < d; ++j) acc += gs[j] * dW[(size_t)i * d + j];
                dKc[(size_t)s * d + i] -= et[s] * acc;       /* g_s dW^T */
            }
            dec[s] -= kdg;
        }
        /* dW now accumulates d/dW_c: the direct path through W_{c+1} is dW itself */

        for (int t = 0; t < n; ++t) {
            const double* qt = Qc + (size_t)t * d;
            const double* dzt = dZ + (size_t)(c0 + t) * d;
            /* recompute hq_t */
            vec_mat(d, d, qt, Wc, hq);
            for (int s = 0; s <= t; ++s) {
                double a = dot(d, qt, Kc + (size_t)s * d) * et[s];
                for (int j = 0; j < d; ++j) hq[j] -= a * G[(size_t)s * d + j];
            }
            /* output stage */
            if (m->kind == KIND_PLAIN) {
                memcpy(dhq, dzt, (size_t)d * sizeof(double));
            } else {
                double r = ln_forward(d, hq, m->gamma, m->beta, m->eps, xh, y);
                ln_backward(d, xh, r, m->gamma, dzt, dhq);
                for (int j = 0; j < d; ++j) {
                    dQc[(size_t)t * d + j] += dzt[j];
                    dgam[j] += dzt[j] * xh[j];
                    dbet[j] += dzt[j];
                }
            }
            /* hq_t = q_t W_c - sum_{s<=t} (q_t . k_s) eta_s g_s */
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int j = 0; j < d; ++j) {
                    acc += dhq[j] * Wc[(size_t)i * d + j];
                    dW[(size_t)i * d + j] += qt[i] * dhq[j];
                }
                dQc[(size_t)t * d + i] += acc;
            }
            for (int s = 0; s <= t; ++s) {
                const double* ks = Kc + (size_t)s * d;
                const double* gs = G + (size_t)s * d;
                double a = dot(d, qt, ks);
                double dcoef = -dot(d, dhq, gs);              /* d/d(a eta_s) */
                for (int j = 0; j < d; ++j) dG[(size_t)s * d + j] -= a * et[s] * dhq[j];
                dec[s] += dcoef * a;
                double da = dcoef * et[s];
                for (int j = 0; j < d; ++j) {
                    dQc[(size_t)t * d + j] += da * ks[j];
                    dKc[(size_t)s * d + j] += da * qt[j];
                }
            }
        }
        /* g_s = d l_s / d h_s at W_c */
        for (int s = 0; s < n; ++s)
            lin_preact_grad_bwd(m, Wc, Kc + (size_t)s * d, Vc + (size_t)s * d, dG + (size_t)s * d, dW,
                                dKc + (size_t)s * d, dVc + (size_t)s * d, dgam, dbet, scratch);
    }
    memcpy(dW0, dW, dd * sizeof(double));
    free(Ws); free(W); free(dW); free(G); free(dG); free(hq); free(dhq);
    free(xh); free(y); free(kd); free(scratch);
}

/* Returns 0 on success, -1 on a bad argument. dZ and dWend may be NULL (zero).
 * dgamma, dbeta ([H,d], summed over the batch) may be NULL for kind PLAIN. */
int ttt_oracle_linear_bwd(int kind, int B, int H, int N, int d, int b, const double* Q, const double* K,
                          const double* V, const double* eta, const double* W0, const double* gamma,
                          const double* beta, double eps, const double* dZ, const double* dWend,
                          double* dQ, double* dK, double* dV, double* deta, double* dW0, double* dgamma,
                          double* dbeta, int nthreads)
{
    if ((kind != KIND_PLAIN && kind != KIND_LN) || B < 1 || H < 1 || N < 1 || d < 1 || b < 1) return -1;
    if (kind == KIND_LN && (!gamma || !beta || !dgamma || !dbeta)) return -1;
    int units = B * H;
    double* zero = NULL;
    if (!dZ) {
        zero = calloc((size_t)units * N * d, sizeof(double));
        dZ = zero;
    }
    double* pg = calloc((size_t)units * d, sizeof(double));
    double* pb = calloc((size_t)units * d, sizeof(double));
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int u = 0; u < units; ++u) {
        int h = u % H;
        lin_model m = {kind, d, kind == KIND_LN ? gamma + (size_t)h * d : NULL,
                       kind == KIND_LN ? beta + (size_t)h * d : NULL, eps};
        size_t so = (size_t)u * N * d, wo = (size_t)u * d * d;
        lin_unit_bwd(&m, N, b, Q + so, K + so, V + so, eta + (size_t)u * N, W0 + wo, dZ + so,
                     dWend ? dWend + wo : NULL, dQ + so, dK + so, dV + so, deta + (size_t)u * N, dW0 + wo,
                     pg + (size_t)u * d, pb + (size_t)u * d);
    }
    if (kind == KIND_LN) {
        memset(dgamma, 0, (size_t)H * d * sizeof(double));
        memset(dbeta, 0, (size_t)H * d * sizeof(double));
        for (int u = 0; u < units; ++u)
            for (int j = 0; j < d; ++j) {
                dgamma[(size_t)(u % H) * d + j] += pg[(size_t)u * d + j];
                dbeta[(size_t)(u % H) * d + j] += pb[(size_t)u * d + j];
            }
    }
    free(pg);
    free(pb);
    free(zero);
    return 0;
}
