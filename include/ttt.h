/*
 * ttt.h -- C ABI of the MI355X (gfx950) TTT-layer forward library, libttt.so.
 *
 * The library computes the forward pass of a Test-Time Training layer in the
 * mini-batch dual form. The layer's recurrent state is the weight set W of a
 * small inner model f. For every mini-batch (chunk) of b tokens the layer takes
 * one gradient-descent step on the per-token loss ||f(k_t; W) - v_t||^2,
 * with every gradient of the chunk taken at the chunk's starting weights W_c,
 * and emits z_t = f(q_t; W_t), where W_t already contains the updates of the
 * chunk's tokens up to and including t.
 *   Web page "Test-Time Training: Linear Complexity Beyond Attention":
 *   section "1. The Self-Supervised Inner-Loop Task" (the loss), section "2. The
 *   Online Gradient Descent Update Rule" (the step), section "3. Forward
 *   Evaluation and Output Projection" (z_t uses the updated W_t), section
 *   "4. Mini-Batch Parallelism (Dual Formulation)" (chunks of b tokens computed
 *   with matrix products that mirror causal attention, the accumulated weight
 *   delta carried from chunk to chunk).
 * In matrix form, per chunk with rows Q, K, V (b x d) and per-token step sizes
 * eta:   G   = d loss / d(pre-activation) at W_c, row by row
 *        Z   = f evaluated on the pre-activation  Q W_c - tril(Q K^T) diag(eta) G
 *        W  <- W_c - K^T diag(eta) G
 * with tril including the diagonal. For f(x) = x W this is
 * Z = Q W_c - 2 tril(Q K^T) diag(eta) E and W_end = W_c - 2 K^T diag(eta) E,
 * E = K W_c - V. The page writes f(k;W) = W k with a loss carrying a factor
 * 1/2; this ABI uses row vectors, f(x;W) = x W, and no 1/2 (the same method
 * with W_page = W^T and eta_page = 2 eta).
 *
 * Conventions shared by every entry point
 *  - All tensor arguments are DEVICE pointers owned by the caller. The library
 *    allocates no memory and keeps no global state; calls are reentrant.
 *  - Token streams Q, K, V: [B, H, N, d], contiguous, d fastest, of dtype
 *    qkv_dtype (TTT_DTYPE_F32 = IEEE fp32, TTT_DTYPE_BF16 = bfloat16).
 *  - eta: [B, H, N] fp32, the step size of each SOURCE token (it scales that
 *    token's own gradient). When eta == NULL every token uses eta_const.
 *  - State: fp32, row index = input feature (f(x) = x W). W_end may equal the
 *    state input (in-place update); any other overlap between an output and an
 *    input is an error.
 *  - Z: [B, H, N, d] fp32 output.
 *  - N need not be a multiple of b: the last chunk holds N mod b tokens.
 *  - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the null
 *    stream). Argument validation happens on the host before any HIP call; a
 *    non-TTT_OK return means nothing was launched. Faults inside kernels surface
 *    at the caller's next synchronisation of the stream. Nothing is printed.
 *  - NaN/Inf in the inputs propagate by IEEE rules; there are no checks on the
 *    hot path.
 */
#ifndef TTT_H_
#define TTT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTT_ABI_VERSION 2

typedef enum {
    TTT_OK = 0,
    TTT_ERR_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, bad enum, bad overlap */
    TTT_ERR_UNSUPPORTED = 2,        /* valid arguments with no kernel for them */
    TTT_ERR_WORKSPACE_TOO_SMALL = 3,
    TTT_ERR_HIP = 4                 /* a HIP launch reported an error */
} ttt_status;

typedef enum { TTT_DTYPE_F32 = 0, TTT_DTYPE_BF16 = 1 } ttt_dtype;

typedef enum {
    TTT_LINEAR_PLAIN = 0,   /* f(x) = x W           (page 1, sec. 1) */
    TTT_LINEAR_LN = 1       /* f(x) = x + LN(x W)   LayerNorm (over d, biased variance,
                               eps inside the square root, fixed gamma/beta) and a
                               residual placed inside the inner model; page 1 sec. 3
                               applies the same pair to the layer output */
} ttt_linear_kind;

typedef enum {
    TTT_PATH_NONE = 0,        /* unsupported combination */
    TTT_PATH_SMALL_B = 1,     /* one workgroup per (sequence, head), state on chip */
    TTT_PATH_LARGE_CHUNK = 2  /* chunk-parallel path for large b (plain f only) */
} ttt_path;

/*
 * ttt_linear_fwd -- TTT-Linear forward, kinds PLAIN and LN.
 *
 *   kind        ttt_linear_kind
 *   qkv_dtype   ttt_dtype of Q, K, V
 *   B, H, N, d  batch, heads, tokens, head dim (all >= 1)
 *   b           mini-batch (chunk) size, >= 1
 *   Q, K, V     device [B,H,N,d] qkv_dtype
 *   eta         device [B,H,N] fp32 or NULL (then eta_const for every token)
 *   W0          device [B,H,d,d] fp32 initial state
 *   ln_gamma    device [H,d] fp32 (kind LN; ignored, may be NULL, for PLAIN)
 *   ln_beta     device [H,d] fp32 (kind LN; ignored, may be NULL, for PLAIN)
 *   ln_eps      LayerNorm epsilon (kind LN), >= 0
 *   Z           device [B,H,N,d] fp32 output
 *   W_end       device [B,H,d,d] fp32 output, the state after the last token;
 *               may equal W0
 *   workspace   device scratch of at least ttt_linear_fwd_workspace_bytes(...)
 *               bytes, 256-byte aligned (may be NULL when that size is 0); it
 *               must not overlap any input or output
 *   hip_stream  hipStream_t to launch on
 * Alignment: Q, K, V, Z and eta 16 bytes; W0, W_end 4 bytes (else
 * TTT_ERR_INVALID_ARGUMENT).
 *
 * Supported (else TTT_ERR_UNSUPPORTED):
 *   small-b path  : kind PLAIN or LN, dtype F32 or BF16, d = 64 or 128,
 *                   1 <= b <= 64 (one workgroup per unit, the state on chip)
 *   large-chunk   : kind PLAIN, dtype F32 or BF16, d = 64 or 128, b > 64, any N.
 *                   With BF16 streams, d = 128, b >= 256, b % 128 == 0,
 *                   N % 128 == 0 and N < 2^22 the chunk-parallel kernels run
 *                   (they need the workspace); every other combination runs one
 *                   workgroup per unit over blocks of 64 tokens (no workspace).
 * ttt_linear_fwd_path() reports which path a combination takes.
 */
int ttt_linear_fwd(int kind, int qkv_dtype, int B, int H, int N, int d, int b,
                   const void* Q, const void* K, const void* V,
                   const float* eta, float eta_const, const float* W0,
                   const float* ln_gamma, const float* ln_beta, float ln_eps,
                   float* Z, float* W_end,
                   void* workspace, size_t workspace_bytes, void* hip_stream);

/* Bytes of device workspace ttt_linear_fwd needs for these sizes (0 for the
 * small-b path). Returns 0 as well for unsupported or invalid combinations. */
size_t ttt_linear_fwd_workspace_bytes(int kind, int qkv_dtype, int B, int H, int N, int d, int b);

/* Size of the library's static device scratch array used by
 * ttt_linear_fwd_noalloc (64 MiB). */
#define TTT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * ttt_linear_fwd_noalloc -- ttt_linear_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). The arguments, results, supported combinations and
 * errors are those of ttt_linear_fwd without the workspace: the large-chunk
 * path puts its workspace in a file-scope device array of
 * TTT_NOALLOC_SCRATCH_BYTES inside the library (one per device, created when
 * the library's code is loaded on that device and kept until the process
 * ends; its address is looked up once per device, on the first call made with
 * that device current). The call allocates nothing and frees nothing.
 *   Returns TTT_ERR_WORKSPACE_TOO_SMALL, before any HIP call, when
 *   ttt_linear_fwd_workspace_bytes(...) exceeds TTT_NOALLOC_SCRATCH_BYTES
 *   (at d = 128: when B*H*(3*ceil(N/b) + 1) exceeds 1024).
 *   Every call on one device shares that device's array and leaves its last
 *   contents there (every byte a call reads it has written first); calls that
 *   overlap in time on one device, on different streams or host threads,
 *   race on it and must be serialised by the caller.
 * The small-b path needs no workspace and runs exactly as ttt_linear_fwd.
 */
int ttt_linear_fwd_noalloc(int kind, int qkv_dtype, int B, int H, int N, int d, int b,
                           const void* Q, const void* K, const void* V,
                           const float* eta, float eta_const, const float* W0,
                           const float* ln_gamma, const float* ln_beta, float ln_eps,
                           float* Z, float* W_end, void* hip_stream);

typedef enum {
    TTT_APPLY_BEFORE_STEP = 0,  /* chunk outputs use the chunk's starting weights W_c */
    TTT_APPLY_AFTER_STEP = 1    /* chunk outputs use the weights after its step, W_{c+1} */
} ttt_block_apply;

/*
 * ttt_linear_fwd_block -- block-causal large-chunk TTT-Linear forward.
 *
 * Page "Test-Time Training Done Right" (abstract) argues for large chunks over
 * small mini-batches with fine-grained block-wise causal dependencies. Read
 * plainly: the state takes one step per chunk with every gradient at the
 * chunk's starting weights (exactly as ttt_linear_fwd, so W_end is the same),
 * and every output of chunk c uses one set of weights, with no causal mask
 * inside the chunk:
 *     apply = TTT_APPLY_BEFORE_STEP:  Z_c = f(Q_c; W_c)
 *     apply = TTT_APPLY_AFTER_STEP:   Z_c = f(Q_c; W_{c+1})
 * Arguments, layouts, ownership, aliasing and errors are those of
 * ttt_linear_fwd; an invalid `apply` is TTT_ERR_INVALID_ARGUMENT.
 * Supported (else TTT_ERR_UNSUPPORTED): the large-chunk combinations of
 * ttt_linear_fwd (kind PLAIN, b > 64, d in {64, 128}, fp32 or bf16 streams, any
 * N). Those that run the chunk-parallel kernels (BF16, d = 128, b >= 256,
 * b % 128 == 0, N % 128 == 0, N < 2^22) take the workspace below; the others
 * need none (ttt_linear_fwd_block_workspace_bytes returns 0 for them).
 */
int ttt_linear_fwd_block(int apply, int kind, int qkv_dtype, int B, int H, int N, int d, int b,
                         const void* Q, const void* K, const void* V,
                         const float* eta, float eta_const, const float* W0,
                         const float* ln_gamma, const float* ln_beta, float ln_eps,
                         float* Z, float* W_end,
                         void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes of ttt_linear_fwd_block (0 for unsupported or invalid input). */
size_t ttt_linear_fwd_block_workspace_bytes(int apply, int kind, int qkv_dtype, int B, int H, int N,
                                            int d, int b);

/*
 * ttt_linear_decode -- one generated token for each of B*H independent
 * (sequence, head) streams: the online rule of page "Test-Time Training:
 * Linear Complexity Beyond Attention" (section "2. The Online Gradient Descent
 * Update Rule", output as in section "3. Forward Evaluation and Output
 * Projection"), i.e. a mini-batch of one token:
 *     g = d ||f(k; W) - v||^2 / d(k W),   W <- W - eta k^T g,   z = f(q; W).
 *
 *   kind        TTT_LINEAR_PLAIN or TTT_LINEAR_LN (conventions of ttt_linear_fwd)
 *   qkv_dtype   dtype of q, k, v
 *   B, H, d     streams = B*H, head dim
 *   q, k, v     device [B,H,d] qkv_dtype
 *   eta         device [B,H] fp32 step size of this token, or NULL (eta_const)
 *   W           device [B,H,d,d] fp32 state, read and overwritten in place
 *   ln_gamma, ln_beta, ln_eps   as for ttt_linear_fwd
 *   z           device [B,H,d] fp32 output
 * W and z must not overlap each other or any input. Asynchronous on hip_stream;
 * validation on the host before any HIP call. Supported: d = 64 (else
 * TTT_ERR_UNSUPPORTED).
 */
int ttt_linear_decode(int kind, int qkv_dtype, int B, int H, int d,
                      const void* q, const void* k, const void* v,
                      const float* eta, float eta_const, float* W,
                      const float* ln_gamma, const float* ln_beta, float ln_eps,
                      float* z, void* hip_stream);

/*
 * ttt_linear_bwd -- backward of ttt_linear_fwd (small-b combinations): the
 * gradients of a scalar objective with respect to every input, given its
 * gradients with respect to the outputs. Page "Test-Time Training: Linear
 * Complexity Beyond Attention" (section "1. The Self-Supervised Inner-Loop
 * Task") trains the outer parameters by backpropagation through the inner
 * loop; this differentiates the chunked computation of section "4. Mini-Batch
 * Parallelism (Dual Formulation)" exactly (every gradient at the chunk-start
 * weights, outputs with the updated weights), including the LayerNorm
 * statistics inside the inner loss and the output.
 *
 *   kind, qkv_dtype, B, H, N, d, b, Q, K, V, eta, eta_const, W0, ln_gamma,
 *   ln_beta, ln_eps      the forward call's arguments (read only)
 *   dZ          device [B,H,N,d] fp32, d objective / d Z
 *   dW_end      device [B,H,d,d] fp32, d objective / d W_end, or NULL (zero)
 *   dQ, dK, dV  device [B,H,N,d] fp32 outputs
 *   deta        device [B,H,N] fp32 output: d objective / d eta_t for every
 *               token (also when eta == NULL: then their sum is the gradient
 *               with respect to eta_const)
 *   dW0         device [B,H,d,d] fp32 output
 *   dgamma, dbeta   device [H,d] fp32 outputs, summed over the batch (kind LN;
 *               ignored, may be NULL, for PLAIN)
 *   workspace   device, 256-byte aligned, ttt_linear_bwd_workspace_bytes(...)
 *               bytes: the chunk-start states (B*H*ceil(N/b)*d*d*4 bytes) and
 *               per-unit partial sums
 * All products run on fp32 matrix cores (exact fp32 products, fp32 sums).
 * Outputs must not overlap each other, any input or the workspace. Pointers of
 * token rows, states, dZ, dW_end, the gradient outputs and ln_gamma/ln_beta
 * must be 16-byte aligned. Asynchronous on hip_stream; validation on the host
 * before any HIP call. Supported: d = 64, 1 <= b <= 16 (else
 * TTT_ERR_UNSUPPORTED).
 */
int ttt_linear_bwd(int kind, int qkv_dtype, int B, int H, int N, int d, int b,
                   const void* Q, const void* K, const void* V,
                   const float* eta, float eta_const, const float* W0,
                   const float* ln_gamma, const float* ln_beta, float ln_eps,
                   const float* dZ, const float* dW_end,
                   float* dQ, float* dK, float* dV, float* deta, float* dW0,
                   float* dgamma, float* dbeta,
                   void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes of ttt_linear_bwd (0 for unsupported or invalid input). */
size_t ttt_linear_bwd_workspace_bytes(int kind, int qkv_dtype, int B, int H, int N, int d, int b);

/* Which ttt_path a (kind, dtype, d, b) combination takes; TTT_PATH_NONE if none. */
int ttt_linear_fwd_path(int kind, int qkv_dtype, int d, int b);

/*
 * ttt_mlp_fwd -- TTT-MLP forward, f(x) = x + LN(GELU(x W1) W2), no biases,
 * GELU(a) = a Phi(a) with the Gaussian CDF Phi = (1 + erf(a / sqrt 2)) / 2 (the
 * erf form, not the tanh approximation). The kernels evaluate erf with
 * Abramowitz & Stegun, "Handbook of Mathematical Functions", formula 7.1.26
 * (|error| <= 1.5e-7, i.e. at most 7.5e-8 in Phi). The page "How to Master
 * Test-Time Training for Infinite Context LLMs" (section "The Math and
 * Architecture of TTT Layers") names a small multi-layer perceptron as the
 * inner model. The dual form is applied to both layers: with A = K W1_c,
 * X2 = GELU(A) and the loss gradients G2 (at the second pre-activation) and
 * G1 = (G2 W2_c^T) * GELU'(A),
 *   A_Q = Q W1_c - tril(Q K^T) diag(eta) G1,  X2_Q = GELU(A_Q),
 *   H_Q = X2_Q W2_c - tril(X2_Q X2^T) diag(eta) G2,  Z = Q + LN(H_Q),
 *   W1 <- W1_c - K^T diag(eta) G1,  W2 <- W2_c - X2^T diag(eta) G2.
 *
 *   hidden      width of the hidden layer (4*d)
 *   W1_0        device [B,H,d,hidden] fp32;  W2_0 device [B,H,hidden,d] fp32
 *   W1_end, W2_end   outputs of the same shapes; may equal W1_0 / W2_0
 *   workspace   device, 256-byte aligned, ttt_mlp_fwd_workspace_bytes(...)
 *               bytes (0, and NULL allowed, for d = 64 with b <= 16, where the
 *               state stays on chip); it must not overlap any other argument
 *   other arguments as for ttt_linear_fwd (ln_gamma/ln_beta required).
 * Alignment: Q, K, V, Z, eta, the states 16 bytes.
 * Supported: dtype F32 or BF16, d = 64 or 128, hidden = 4 d, 1 <= b <= 64
 * (else TTT_ERR_UNSUPPORTED). For d = 64 and b <= 16 the state stays in MFMA
 * accumulators for the whole scan; otherwise it lives in the workspace (and
 * W2_end), read and written once per chunk.
 */
int ttt_mlp_fwd(int qkv_dtype, int B, int H, int N, int d, int hidden, int b,
                const void* Q, const void* K, const void* V,
                const float* eta, float eta_const,
                const float* W1_0, const float* W2_0,
                const float* ln_gamma, const float* ln_beta, float ln_eps,
                float* Z, float* W1_end, float* W2_end,
                void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes of ttt_mlp_fwd (0 when none is needed, and for unsupported
 * or invalid input). */
size_t ttt_mlp_fwd_workspace_bytes(int qkv_dtype, int B, int H, int N, int d, int hidden, int b);

/*
 * ttt_layer_fwd -- the whole TTT layer around TTT-Linear: projections, key
 * normalisation, the inner model, and the output stage. Page "Test-Time
 * Training: Linear Complexity Beyond Attention": section "1. The
 * Self-Supervised Inner-Loop Task" (q, k, v are linear projections of the
 * token), the page's layer code (keys scaled to unit L2 length before the
 * inner loop), section "3. Forward Evaluation and Output Projection"
 * (y = W_O (LayerNorm(z) + q)). Per token x_t (width D) and head h:
 *     q = W_Q x,  k = W_K x / ||W_K x||,  v = W_V x   (head h: outputs h*d .. h*d+d-1;
 *                                                     a zero key stays zero)
 *     z = the inner model of ttt_linear_fwd (kind, chunks of b, eta, W0)
 *     y = W_O (LayerNorm(z) * out_gamma + out_beta + q)   (LayerNorm per head)
 *
 *   kind            TTT_LINEAR_PLAIN or TTT_LINEAR_LN (the inner model)
 *   B, N, D         sequences, tokens per sequence, model width
 *   H, d            heads and head width (H*d projection outputs)
 *   b               chunk length of the inner model
 *   x               device [B, N, D] bf16 tokens
 *   Wq, Wk, Wv      device [H*d, D] bf16 (output-major: row o holds the
 *                   weights of projection output o, as q = W_Q x reads)
 *   Wo              device [D, H*d] bf16 (row n: weights of model output n)
 *   eta, eta_const  step sizes as for ttt_linear_fwd ([B, H, N] or NULL)
 *   W0, W_end       device [B, H, d, d] fp32 inner state in / out (may be equal)
 *   ln_gamma, ln_beta   [H, d] fp32 inner LayerNorm (kind LN only, else unused)
 *   out_gamma, out_beta [H, d] fp32 output LayerNorm affine, 16-byte aligned
 *   ln_eps          epsilon of both LayerNorms (biased variance, inside the root)
 *   y               device [B, N, D] fp32 output
 *   workspace       device, 256-byte aligned, at least
 *                   ttt_layer_fwd_workspace_bytes(B, N, H, d) bytes = 5 S,
 *                   S = B*H*N*d*4 rounded up to a multiple of 256. On return it
 *                   holds Q, K (normalised), V and Z at offsets 0, S, 2S, 3S; the
 *                   last S bytes are scratch. Q, K and V are each two bf16
 *                   [B, H, N, d] planes, the second starting B*H*N*d*2 bytes after
 *                   the first: the RNE rounding of the fp32 value and the rounding
 *                   of the remainder (their sum carries 16 significant bits); Z is
 *                   fp32 [B, H, N, d].
 * x and the four weights must be 16-byte aligned. y, W_end and the workspace
 * must not overlap any input or each other (W_end may equal W0). Products run
 * on bf16 matrix cores with fp32 accumulation; the projected fp32 streams, the
 * inner state and its gradients, and the LayerNorm output entering W_O's
 * product are carried as two bf16 terms (16 significant bits). Asynchronous on hip_stream;
 * validation on the host before any HIP call.
 * Supported: d = 64, 1 <= b <= 16, D a multiple of 64, B*H*N < 2^27 (else
 * TTT_ERR_UNSUPPORTED).
 */
int ttt_layer_fwd(int kind, int B, int N, int D, int H, int d, int b,
                  const void* x, const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                  const float* eta, float eta_const, const float* W0,
                  const float* ln_gamma, const float* ln_beta,
                  const float* out_gamma, const float* out_beta, float ln_eps,
                  float* y, float* W_end, void* workspace, size_t workspace_bytes,
                  void* hip_stream);

/* Workspace bytes of ttt_layer_fwd (0 for invalid sizes). */
size_t ttt_layer_fwd_workspace_bytes(int B, int N, int H, int d);

/* Static, NUL-terminated description of a ttt_status value. */
const char* ttt_status_string(int status);

/* TTT_ABI_VERSION of the built library. */
int ttt_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H_ */
