/*
 * ttt_oracle.c -- slow, plain fp64 CPU oracle for the TTT-layer forward pass.
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
