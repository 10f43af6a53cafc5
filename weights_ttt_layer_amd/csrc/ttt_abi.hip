// ttt_abi.hip -- the extern "C" entry points declared in include/ttt.h:
// synchronous host-side validation, path selection and kernel launch.
// Validation touches no HIP API, so every rejection path is testable on a
// machine without a GPU.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/ttt.h"
#include "kernels.h"

namespace {

constexpr int SMALLB_D = 64;
constexpr int SMALLB_MAX_B = 16;       // the backward, decode and whole-layer paths
constexpr int SMALLB_D2 = 128;         // the forward small-b path also takes d = 128
constexpr int SMALLB_FWD_MAX_B = 64;   // ... and chunks of up to 64 tokens
constexpr int LARGE_D = 128;
constexpr int LARGE_MIN_B = 256;
constexpr int LARGE_B_MULT = 128;
constexpr int LARGE_MAX_N = 1 << 22;   // Z rows of one unit addressed with 32-bit byte offsets

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [a, a+na) and [b, b+nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int linear_path(int kind, int dtype, int d, int b)
{
    const bool kinds = kind == TTT_LINEAR_PLAIN || kind == TTT_LINEAR_LN;
    const bool dtypes = dtype == TTT_DTYPE_F32 || dtype == TTT_DTYPE_BF16;
    if (!kinds || !dtypes || (d != SMALLB_D && d != SMALLB_D2) || b < 1) return TTT_PATH_NONE;
    if (b <= SMALLB_FWD_MAX_B) return TTT_PATH_SMALL_B;
    if (kind == TTT_LINEAR_PLAIN) return TTT_PATH_LARGE_CHUNK;   // longer chunks: plain f
    return TTT_PATH_NONE;
}

// The chunk-parallel large-chunk kernels (a workspace, three launches) take bf16
// streams at d = 128 with b and N multiples of 128; every other large-chunk
// combination runs the generic kernel's block mode (one workgroup per unit,
// no workspace).
bool fast_large(int dtype, int d, int b, int N)
{
    return dtype == TTT_DTYPE_BF16 && d == LARGE_D && b >= LARGE_MIN_B && b % LARGE_B_MULT == 0 &&
           N % LARGE_B_MULT == 0 && N < LARGE_MAX_N;
}

size_t elem_size(int dtype) { return dtype == TTT_DTYPE_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

int ttt_abi_version(void) { return TTT_ABI_VERSION; }

const char* ttt_status_string(int status)
{
    switch (status) {
        case TTT_OK: return "TTT_OK: success";
        case TTT_ERR_INVALID_ARGUMENT: return "TTT_ERR_INVALID_ARGUMENT: invalid argument";
        case TTT_ERR_UNSUPPORTED: return "TTT_ERR_UNSUPPORTED: no kernel for this combination";
        case TTT_ERR_WORKSPACE_TOO_SMALL: return "TTT_ERR_WORKSPACE_TOO_SMALL: workspace too small";
        case TTT_ERR_HIP: return "TTT_ERR_HIP: a HIP launch failed";
        default: return "unknown ttt_status";
    }
}

int ttt_linear_fwd_path(int kind, int qkv_dtype, int d, int b) { return linear_path(kind, qkv_dtype, d, b); }

size_t ttt_linear_fwd_workspace_bytes(int kind, int qkv_dtype, int B, int H, int N, int d, int b)
{
    if (B < 1 || H < 1 || N < 1 || d < 1 || b < 1) return 0;
    if (linear_path(kind, qkv_dtype, d, b) != TTT_PATH_LARGE_CHUNK || !fast_large(qkv_dtype, d, b, N)) return 0;
    return ttt::large_chunk_workspace_bytes(B, H, N, d, b);
}

}  // extern "C"

namespace {

// Validation shared by the chunked forward entry points; fills `a` and the
// path on success. Touches no HIP API.
int check_linear(int kind, int qkv_dtype, int B, int H, int N, int d, int b, const void* Q, const void* K,
                 const void* V, const float* eta, float eta_const, const float* W0, const float* ln_gamma,
                 const float* ln_beta, float ln_eps, float* Z, float* W_end, void* workspace,
                 size_t workspace_bytes, ttt::LinearArgs& a, int& path, bool internal_workspace = false)
{
    if (kind != TTT_LINEAR_PLAIN && kind != TTT_LINEAR_LN) return TTT_ERR_INVALID_ARGUMENT;
    if (qkv_dtype != TTT_DTYPE_F32 && qkv_dtype != TTT_DTYPE_BF16) return TTT_ERR_INVALID_ARGUMENT;
    if (B < 1 || H < 1 || N < 1 || d < 1 || b < 1) return TTT_ERR_INVALID_ARGUMENT;
    if (!Q || !K || !V || !W0 || !Z || !W_end) return TTT_ERR_INVALID_ARGUMENT;
    if (kind == TTT_LINEAR_LN && (!ln_gamma || !ln_beta || !(ln_eps >= 0.f)))
        return TTT_ERR_INVALID_ARGUMENT;
    // Z rows leave as 16-byte stores; per-token eta is read in 16-byte vectors
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(W0, 4) ||
        !aligned(Z, 16) || !aligned(W_end, 4) || (eta && !aligned(eta, 16)))
        return TTT_ERR_INVALID_ARGUMENT;
    // size arithmetic in 64 bits; reject overflow of the int32 sizes' products
    const size_t units = (size_t)B * (size_t)H;
    const size_t tok = units * (size_t)N;
    const size_t qkv_bytes = tok * (size_t)d * elem_size(qkv_dtype);
    const size_t z_bytes = tok * (size_t)d * 4;
    const size_t w_bytes = units * (size_t)d * (size_t)d * 4;
    if (units > (size_t)INT32_MAX || tok / units != (size_t)N) return TTT_ERR_INVALID_ARGUMENT;
    // Z must not overlap any input; W_end must equal W0 or not overlap it
    if (overlaps(Z, z_bytes, Q, qkv_bytes) || overlaps(Z, z_bytes, K, qkv_bytes) ||
        overlaps(Z, z_bytes, V, qkv_bytes) || overlaps(Z, z_bytes, W0, w_bytes) ||
        overlaps(Z, z_bytes, W_end, w_bytes) || (eta && overlaps(Z, z_bytes, eta, tok * 4)))
        return TTT_ERR_INVALID_ARGUMENT;
    if (W_end != W0 && overlaps(W_end, w_bytes, W0, w_bytes)) return TTT_ERR_INVALID_ARGUMENT;
    if (overlaps(W_end, w_bytes, Q, qkv_bytes) || overlaps(W_end, w_bytes, K, qkv_bytes) ||
        overlaps(W_end, w_bytes, V, qkv_bytes) || (eta && overlaps(W_end, w_bytes, eta, tok * 4)))
        return TTT_ERR_INVALID_ARGUMENT;

    path = linear_path(kind, qkv_dtype, d, b);
    if (path == TTT_PATH_NONE) return TTT_ERR_UNSUPPORTED;
    if (path == TTT_PATH_LARGE_CHUNK && fast_large(qkv_dtype, d, b, N) && !internal_workspace) {
        const size_t need = ttt::large_chunk_workspace_bytes(B, H, N, d, b);
        if (workspace_bytes < need || (need > 0 && !workspace)) return TTT_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned(workspace, 256)) return TTT_ERR_INVALID_ARGUMENT;
        if (overlaps(workspace, need, Z, z_bytes) || overlaps(workspace, need, W_end, w_bytes) ||
            overlaps(workspace, need, Q, qkv_bytes) || overlaps(workspace, need, K, qkv_bytes) ||
            overlaps(workspace, need, V, qkv_bytes) || overlaps(workspace, need, W0, w_bytes) ||
            (eta && overlaps(workspace, need, eta, tok * 4)))
            return TTT_ERR_INVALID_ARGUMENT;
    }

    a.kind = kind;
    a.dtype = qkv_dtype;
    a.B = B;
    a.H = H;
    a.N = N;
    a.d = d;
    a.b = b;
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.eta = eta;
    a.eta_const = eta_const;
    a.W0 = W0;
    a.gamma = ln_gamma;
    a.beta = ln_beta;
    a.eps = ln_eps;
    a.Z = Z;
    a.W_end = W_end;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    return TTT_OK;
}

}  // namespace

extern "C" {

int ttt_linear_fwd(int kind, int qkv_dtype, int B, int H, int N, int d, int b, const void* Q,
                   const void* K, const void* V, const float* eta, float eta_const, const float* W0,
                   const float* ln_gamma, const float* ln_beta, float ln_eps, float* Z, float* W_end,
                   void* workspace, size_t workspace_bytes, void* hip_stream)
{
    ttt::LinearArgs a;
    int path = TTT_PATH_NONE;
    const int st = check_linear(kind, qkv_dtype, B, H, N, d, b, Q, K, V, eta, eta_const, W0, ln_gamma, ln_beta,
                                ln_eps, Z, W_end, workspace, workspace_bytes, a, path);
    if (st != TTT_OK) return st;
    hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
    hipError_t err;
    if (path == TTT_PATH_SMALL_B)
        err = ttt::launch_smallb_linear(a, stream);
    else if (fast_large(qkv_dtype, d, b, N))
        err = ttt::launch_large_chunk_linear(a, ttt::LC_OUT_DUAL, stream);
    else
        err = ttt::launch_midb_linear_blocks(a, ttt::LC_OUT_DUAL, stream);
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

size_t ttt_linear_fwd_block_workspace_bytes(int apply, int kind, int qkv_dtype, int B, int H, int N, int d, int b)
{
    if (apply != TTT_APPLY_BEFORE_STEP && apply != TTT_APPLY_AFTER_STEP) return 0;
    return ttt_linear_fwd_workspace_bytes(kind, qkv_dtype, B, H, N, d, b);
}

int ttt_linear_fwd_block(int apply, int kind, int qkv_dtype, int B, int H, int N, int d, int b, const void* Q,
                         const void* K, const void* V, const float* eta, float eta_const, const float* W0,
                         const float* ln_gamma, const float* ln_beta, float ln_eps, float* Z, float* W_end,
                         void* workspace, size_t workspace_bytes, void* hip_stream)
{
    if (apply != TTT_APPLY_BEFORE_STEP && apply != TTT_APPLY_AFTER_STEP) return TTT_ERR_INVALID_ARGUMENT;
    ttt::LinearArgs a;
    int path = TTT_PATH_NONE;
    const int st = check_linear(kind, qkv_dtype, B, H, N, d, b, Q, K, V, eta, eta_const, W0, ln_gamma, ln_beta,
                                ln_eps, Z, W_end, workspace, workspace_bytes, a, path);
    if (st != TTT_OK) return st;
    if (path != TTT_PATH_LARGE_CHUNK) return TTT_ERR_UNSUPPORTED;
    const int outputs = apply == TTT_APPLY_BEFORE_STEP ? ttt::LC_OUT_BEFORE : ttt::LC_OUT_AFTER;
    hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
    const hipError_t err = fast_large(qkv_dtype, d, b, N) ? ttt::launch_large_chunk_linear(a, outputs, stream)
                                                          : ttt::launch_midb_linear_blocks(a, outputs, stream);
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

int ttt_linear_decode(int kind, int qkv_dtype, int B, int H, int d, const void* q, const void* k, const void* v,
                      const float* eta, float eta_const, float* W, const float* ln_gamma, const float* ln_beta,
                      float ln_eps, float* z, void* hip_stream)
{
    if (kind != TTT_LINEAR_PLAIN && kind != TTT_LINEAR_LN) return TTT_ERR_INVALID_ARGUMENT;
    if (qkv_dtype != TTT_DTYPE_F32 && qkv_dtype != TTT_DTYPE_BF16) return TTT_ERR_INVALID_ARGUMENT;
    if (B < 1 || H < 1 || d < 1) return TTT_ERR_INVALID_ARGUMENT;
    if (!q || !k || !v || !W || !z) return TTT_ERR_INVALID_ARGUMENT;
    if (kind == TTT_LINEAR_LN && (!ln_gamma || !ln_beta || !(ln_eps >= 0.f))) return TTT_ERR_INVALID_ARGUMENT;
    const size_t es = elem_size(qkv_dtype);
    if (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(W, 4) || !aligned(z, 4) ||
        (eta && !aligned(eta, 4)))
        return TTT_ERR_INVALID_ARGUMENT;
    const size_t units = (size_t)B * (size_t)H;
    if (units > (size_t)INT32_MAX) return TTT_ERR_INVALID_ARGUMENT;
    const size_t vec_bytes = units * (size_t)d * es;
    const size_t z_bytes = units * (size_t)d * 4;
    const size_t w_bytes = units * (size_t)d * (size_t)d * 4;
    const void* ins[3] = {q, k, v};
    for (int i = 0; i < 3; ++i)
        if (overlaps(z, z_bytes, ins[i], vec_bytes) || overlaps(W, w_bytes, ins[i], vec_bytes))
            return TTT_ERR_INVALID_ARGUMENT;
    if (overlaps(z, z_bytes, W, w_bytes) || (eta && (overlaps(z, z_bytes, eta, units * 4) ||
                                                     overlaps(W, w_bytes, eta, units * 4))))
        return TTT_ERR_INVALID_ARGUMENT;
    if (d != SMALLB_D) return TTT_ERR_UNSUPPORTED;

    ttt::LinearArgs a{};
    a.kind = kind;
    a.dtype = qkv_dtype;
    a.B = B;
    a.H = H;
    a.N = 1;
    a.d = d;
    a.b = 1;
    a.Q = q;
    a.K = k;
    a.V = v;
    a.eta = eta;
    a.eta_const = eta_const;
    a.W0 = W;
    a.gamma = ln_gamma;
    a.beta = ln_beta;
    a.eps = ln_eps;
    a.Z = z;
    a.W_end = W;
    const hipError_t err = ttt::launch_decode_linear(a, reinterpret_cast<hipStream_t>(hip_stream));
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

size_t ttt_mlp_fwd_workspace_bytes(int qkv_dtype, int B, int H, int N, int d, int hidden, int b)
{
    if (qkv_dtype != TTT_DTYPE_F32 && qkv_dtype != TTT_DTYPE_BF16) return 0;
    if (B < 1 || H < 1 || N < 1 || b < 1) return 0;
    if (!((d == 64 || d == 128) && hidden == 4 * d && b <= 64)) return 0;
    if ((size_t)B * (size_t)H > (size_t)INT32_MAX) return 0;
    if (d == 64 && b <= 16) return 0;   // the state stays in registers
    return ttt::mlp_generic_workspace_bytes(B, H, d, b);
}

int ttt_mlp_fwd(int qkv_dtype, int B, int H, int N, int d, int hidden, int b, const void* Q,
                const void* K, const void* V, const float* eta, float eta_const, const float* W1_0,
                const float* W2_0, const float* ln_gamma, const float* ln_beta, float ln_eps,
                float* Z, float* W1_end, float* W2_end, void* workspace, size_t workspace_bytes,
                void* hip_stream)
{
    if (qkv_dtype != TTT_DTYPE_F32 && qkv_dtype != TTT_DTYPE_BF16) return TTT_ERR_INVALID_ARGUMENT;
    if (B < 1 || H < 1 || N < 1 || d < 1 || hidden < 1 || b < 1) return TTT_ERR_INVALID_ARGUMENT;
    if (!Q || !K || !V || !W1_0 || !W2_0 || !ln_gamma || !ln_beta || !Z || !W1_end || !W2_end)
        return TTT_ERR_INVALID_ARGUMENT;
    if (!(ln_eps >= 0.f)) return TTT_ERR_INVALID_ARGUMENT;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(W1_0, 16) ||
        !aligned(W2_0, 16) || !aligned(Z, 16) || !aligned(W1_end, 16) || !aligned(W2_end, 16) ||
        (eta && !aligned(eta, 16)))
        return TTT_ERR_INVALID_ARGUMENT;
    const size_t units = (size_t)B * (size_t)H;
    const size_t tok = units * (size_t)N;
    const size_t qkv_bytes = tok * (size_t)d * elem_size(qkv_dtype);
    const size_t z_bytes = tok * (size_t)d * 4;
    const size_t w_bytes = units * (size_t)d * (size_t)hidden * 4;
    if (units > (size_t)INT32_MAX) return TTT_ERR_INVALID_ARGUMENT;
    const void* ins[5] = {Q, K, V, W1_0, W2_0};
    const size_t in_bytes[5] = {qkv_bytes, qkv_bytes, qkv_bytes, w_bytes, w_bytes};
    for (int i = 0; i < 5; ++i) {
        if (overlaps(Z, z_bytes, ins[i], in_bytes[i])) return TTT_ERR_INVALID_ARGUMENT;
        if (i < 3 && (overlaps(W1_end, w_bytes, ins[i], in_bytes[i]) ||
                      overlaps(W2_end, w_bytes, ins[i], in_bytes[i])))
            return TTT_ERR_INVALID_ARGUMENT;
    }
    if (eta && (overlaps(Z, z_bytes, eta, tok * 4) || overlaps(W1_end, w_bytes, eta, tok * 4) ||
                overlaps(W2_end, w_bytes, eta, tok * 4)))
        return TTT_ERR_INVALID_ARGUMENT;
    if (overlaps(Z, z_bytes, W1_end, w_bytes) || overlaps(Z, z_bytes, W2_end, w_bytes) ||
        overlaps(W1_end, w_bytes, W2_end, w_bytes))
        return TTT_ERR_INVALID_ARGUMENT;
    if (W1_end != W1_0 && overlaps(W1_end, w_bytes, W1_0, w_bytes)) return TTT_ERR_INVALID_ARGUMENT;
    if (W2_end != W2_0 && overlaps(W2_end, w_bytes, W2_0, w_bytes)) return TTT_ERR_INVALID_ARGUMENT;
    if (overlaps(W1_end, w_bytes, W2_0, w_bytes) || overlaps(W2_end, w_bytes, W1_0, w_bytes))
        return TTT_ERR_INVALID_ARGUMENT;

    if (!((d == 64 || d == 128) && hidden == 4 * d && b <= 64)) return TTT_ERR_UNSUPPORTED;
    const size_t need = ttt_mlp_fwd_workspace_bytes(qkv_dtype, B, H, N, d, hidden, b);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return TTT_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned(workspace, 256)) return TTT_ERR_INVALID_ARGUMENT;
        const void* others[9] = {Q, K, V, W1_0, W2_0, Z, W1_end, W2_end, eta};
        const size_t other_bytes[9] = {qkv_bytes, qkv_bytes, qkv_bytes, w_bytes, w_bytes, z_bytes, w_bytes, w_bytes,
                                       eta ? tok * 4 : 0};
        for (int i = 0; i < 9; ++i)
            if (overlaps(workspace, need, others[i], other_bytes[i])) return TTT_ERR_INVALID_ARGUMENT;
    }

    ttt::MlpArgs a;
    a.dtype = qkv_dtype;
    a.B = B;
    a.H = H;
    a.N = N;
    a.d = d;
    a.hidden = hidden;
    a.b = b;
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.eta = eta;
    a.eta_const = eta_const;
    a.W1 = W1_0;
    a.W2 = W2_0;
    a.gamma = ln_gamma;
    a.beta = ln_beta;
    a.eps = ln_eps;
    a.Z = Z;
    a.W1_end = W1_end;
    a.W2_end = W2_end;
    hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
    const hipError_t err = need == 0 ? ttt::launch_smallb_mlp(a, stream) : ttt::launch_mlp_generic(a, workspace, stream);
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

size_t ttt_layer_fwd_workspace_bytes(int B, int N, int H, int d)
{
    if (B < 1 || N < 1 || H < 1 || d != SMALLB_D) return 0;
    if ((size_t)B * (size_t)H > (size_t)INT32_MAX) return 0;
    return 5 * ttt::layer_workspace_region_bytes(B, N, H);
}

int ttt_layer_fwd(int kind, int B, int N, int D, int H, int d, int b, const void* x, const void* Wq,
                  const void* Wk, const void* Wv, const void* Wo, const float* eta, float eta_const,
                  const float* W0, const float* ln_gamma, const float* ln_beta, const float* out_gamma,
                  const float* out_beta, float ln_eps, float* y, float* W_end, void* workspace,
                  size_t workspace_bytes, void* hip_stream)
{
    if (kind != TTT_LINEAR_PLAIN && kind != TTT_LINEAR_LN) return TTT_ERR_INVALID_ARGUMENT;
    if (B < 1 || N < 1 || D < 1 || H < 1 || d < 1 || b < 1) return TTT_ERR_INVALID_ARGUMENT;
    if (!x || !Wq || !Wk || !Wv || !Wo || !W0 || !out_gamma || !out_beta || !y || !W_end || !workspace)
        return TTT_ERR_INVALID_ARGUMENT;
    if (!(ln_eps >= 0.f)) return TTT_ERR_INVALID_ARGUMENT;
    if (!aligned(x, 16) || !aligned(Wq, 16) || !aligned(Wk, 16) || !aligned(Wv, 16) || !aligned(Wo, 16) ||
        !aligned(out_gamma, 16) || !aligned(out_beta, 16) || !aligned(y, 4) || !aligned(workspace, 256))
        return TTT_ERR_INVALID_ARGUMENT;
    if ((size_t)B * (size_t)H > (size_t)INT32_MAX || (size_t)B * (size_t)N > (size_t)INT32_MAX)
        return TTT_ERR_INVALID_ARGUMENT;
    if (d != SMALLB_D || b > SMALLB_MAX_B || D % 64 != 0 || (size_t)H * d * 3 > (size_t)INT32_MAX)
        return TTT_ERR_UNSUPPORTED;
    // the output-operand kernel gives each (token, head) row 16 threads of a 32-bit grid
    if ((size_t)B * H * N * 16 > (size_t)INT32_MAX) return TTT_ERR_UNSUPPORTED;
    const size_t region = ttt::layer_workspace_region_bytes(B, N, H);
    if (workspace_bytes < 5 * region) return TTT_ERR_WORKSPACE_TOO_SMALL;

    const size_t HD = (size_t)H * d;
    const size_t x_bytes = (size_t)B * N * D * 2, y_bytes = (size_t)B * N * D * 4;
    const size_t wp_bytes = HD * (size_t)D * 2, w_bytes = (size_t)B * H * d * d * 4;
    const size_t hv_bytes = HD * 4, eta_bytes = (size_t)B * H * N * 4;
    const void* ins[8] = {x, Wq, Wk, Wv, Wo, W0, out_gamma, out_beta};
    const size_t in_bytes[8] = {x_bytes, wp_bytes, wp_bytes, wp_bytes, wp_bytes, w_bytes, hv_bytes, hv_bytes};
    for (int i = 0; i < 8; ++i) {
        if (overlaps(y, y_bytes, ins[i], in_bytes[i]) || overlaps(workspace, 5 * region, ins[i], in_bytes[i]))
            return TTT_ERR_INVALID_ARGUMENT;
        if (i != 5 && overlaps(W_end, w_bytes, ins[i], in_bytes[i])) return TTT_ERR_INVALID_ARGUMENT;
    }
    if (W_end != W0 && overlaps(W_end, w_bytes, W0, w_bytes)) return TTT_ERR_INVALID_ARGUMENT;
    if (overlaps(y, y_bytes, W_end, w_bytes) || overlaps(y, y_bytes, workspace, 5 * region) ||
        overlaps(W_end, w_bytes, workspace, 5 * region))
        return TTT_ERR_INVALID_ARGUMENT;
    if (eta && (overlaps(y, y_bytes, eta, eta_bytes) || overlaps(W_end, w_bytes, eta, eta_bytes) ||
                overlaps(workspace, 5 * region, eta, eta_bytes)))
        return TTT_ERR_INVALID_ARGUMENT;

    char* ws = static_cast<char*>(workspace);
    // Q, K, V: two bf16 planes each (hi, then lo); Z fp32
    uint16_t* Qf = reinterpret_cast<uint16_t*>(ws);
    uint16_t* Kf = reinterpret_cast<uint16_t*>(ws + region);
    uint16_t* Vf = reinterpret_cast<uint16_t*>(ws + 2 * region);
    float* Zf = reinterpret_cast<float*>(ws + 3 * region);
    void* Aext = ws + 4 * region;
    ttt::LinearArgs inner;
    int path = TTT_PATH_NONE;
    const int st = check_linear(kind, TTT_DTYPE_F32, B, H, N, d, b, Qf, Kf, Vf, eta, eta_const, W0, ln_gamma,
                                ln_beta, ln_eps, Zf, W_end, nullptr, 0, inner, path);
    if (st != TTT_OK) return st;
    if (path != TTT_PATH_SMALL_B) return TTT_ERR_UNSUPPORTED;

    ttt::LayerArgs a;
    a.B = B;
    a.N = N;
    a.D = D;
    a.H = H;
    a.x = x;
    a.Wq = Wq;
    a.Wk = Wk;
    a.Wv = Wv;
    a.Wo = Wo;
    a.out_gamma = out_gamma;
    a.out_beta = out_beta;
    a.eps = ln_eps;
    a.y = y;
    hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
    hipError_t err = ttt::launch_layer_qkv(a, Qf, Kf, Vf, stream);
    if (err == hipSuccess) err = ttt::launch_smallb_chain_terms2(inner, stream);
    if (err == hipSuccess) err = ttt::launch_layer_out(a, Zf, Qf, Aext, stream);
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

size_t ttt_linear_bwd_workspace_bytes(int kind, int qkv_dtype, int B, int H, int N, int d, int b)
{
    if (kind != TTT_LINEAR_PLAIN && kind != TTT_LINEAR_LN) return 0;
    if (qkv_dtype != TTT_DTYPE_F32 && qkv_dtype != TTT_DTYPE_BF16) return 0;
    if (B < 1 || H < 1 || N < 1 || d != SMALLB_D || b < 1 || b > SMALLB_MAX_B) return 0;
    if ((size_t)B * (size_t)H > (size_t)INT32_MAX) return 0;
    return ttt::bwd_workspace_bytes(B, H, N, b);
}

int ttt_linear_bwd(int kind, int qkv_dtype, int B, int H, int N, int d, int b, const void* Q, const void* K,
                   const void* V, const float* eta, float eta_const, const float* W0, const float* ln_gamma,
                   const float* ln_beta, float ln_eps, const float* dZ, const float* dW_end, float* dQ, float* dK,
                   float* dV, float* deta, float* dW0, float* dgamma, float* dbeta, void* workspace,
                   size_t workspace_bytes, void* hip_stream)
{
    if (kind != TTT_LINEAR_PLAIN && kind != TTT_LINEAR_LN) return TTT_ERR_INVALID_ARGUMENT;
    if (qkv_dtype != TTT_DTYPE_F32 && qkv_dtype != TTT_DTYPE_BF16) return TTT_ERR_INVALID_ARGUMENT;
    if (B < 1 || H < 1 || N < 1 || d < 1 || b < 1) return TTT_ERR_INVALID_ARGUMENT;
    if (!Q || !K || !V || !W0 || !dZ || !dQ || !dK || !dV || !deta || !dW0 || !workspace)
        return TTT_ERR_INVALID_ARGUMENT;
    const bool ln = kind == TTT_LINEAR_LN;
    if (ln && (!ln_gamma || !ln_beta || !dgamma || !dbeta || !(ln_eps >= 0.f))) return TTT_ERR_INVALID_ARGUMENT;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(W0, 16) || !aligned(dZ, 16) ||
        (dW_end && !aligned(dW_end, 16)) || !aligned(dQ, 16) || !aligned(dK, 16) || !aligned(dV, 16) ||
        !aligned(deta, 4) || !aligned(dW0, 16) || (eta && !aligned(eta, 4)) || !aligned(workspace, 256))
        return TTT_ERR_INVALID_ARGUMENT;
    if (ln && (!aligned(ln_gamma, 16) || !aligned(ln_beta, 16) || !aligned(dgamma, 4) || !aligned(dbeta, 4)))
        return TTT_ERR_INVALID_ARGUMENT;
    const size_t units = (size_t)B * (size_t)H;
    const size_t tok = units * (size_t)N;
    if (units > (size_t)INT32_MAX || tok / units != (size_t)N) return TTT_ERR_INVALID_ARGUMENT;
    if (d != SMALLB_D || b > SMALLB_MAX_B) return TTT_ERR_UNSUPPORTED;
    const size_t need = ttt::bwd_workspace_bytes(B, H, N, b);
    if (workspace_bytes < need) return TTT_ERR_WORKSPACE_TOO_SMALL;

    const size_t qkv_bytes = tok * (size_t)d * elem_size(qkv_dtype), f_bytes = tok * (size_t)d * 4;
    const size_t w_bytes = units * (size_t)d * (size_t)d * 4, e_bytes = tok * 4, hv_bytes = (size_t)H * d * 4;
    // outputs: disjoint from each other, from every input and from the workspace
    const void* outs[7] = {dQ, dK, dV, deta, dW0, ln ? dgamma : nullptr, ln ? dbeta : nullptr};
    const size_t out_bytes[7] = {f_bytes, f_bytes, f_bytes, e_bytes, w_bytes, hv_bytes, hv_bytes};
    const void* ins[10] = {Q, K, V, eta, W0, ln ? ln_gamma : nullptr, ln ? ln_beta : nullptr, dZ, dW_end, workspace};
    const size_t in_bytes[10] = {qkv_bytes, qkv_bytes, qkv_bytes, e_bytes, w_bytes, hv_bytes, hv_bytes, f_bytes,
                                 w_bytes, need};
    for (int i = 0; i < 7; ++i) {
        for (int j = 0; j < 10; ++j)
            if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return TTT_ERR_INVALID_ARGUMENT;
        for (int j = i + 1; j < 7; ++j)
            if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return TTT_ERR_INVALID_ARGUMENT;
    }
    for (int j = 0; j < 9; ++j)
        if (overlaps(workspace, need, ins[j], in_bytes[j])) return TTT_ERR_INVALID_ARGUMENT;

    ttt::BwdArgs a{};
    a.f.kind = kind;
    a.f.dtype = qkv_dtype;
    a.f.B = B;
    a.f.H = H;
    a.f.N = N;
    a.f.d = d;
    a.f.b = b;
    a.f.Q = Q;
    a.f.K = K;
    a.f.V = V;
    a.f.eta = eta;
    a.f.eta_const = eta_const;
    a.f.W0 = W0;
    a.f.gamma = ln_gamma;
    a.f.beta = ln_beta;
    a.f.eps = ln_eps;
    a.f.workspace = workspace;
    a.f.workspace_bytes = workspace_bytes;
    a.dZ = dZ;
    a.dW_end = dW_end;
    a.dQ = dQ;
    a.dK = dK;
    a.dV = dV;
    a.deta = deta;
    a.dW0 = dW0;
    a.dgamma = dgamma;
    a.dbeta = dbeta;
    const hipError_t err = ttt::launch_bwd_linear(a, reinterpret_cast<hipStream_t>(hip_stream));
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// ttt_linear_fwd_noalloc: ttt_linear_fwd with its workspace in a file-scope
// device array instead of a caller buffer, for callers that cannot allocate.
// ---------------------------------------------------------------------------
namespace {

// One copy per device, created when the code object is loaded on that device
// and held until the process ends. In host code `scratch` names a host-side
// stand-in: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) char scratch[TTT_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of `scratch` on the current device, looked up once per device.
hipError_t scratch_on_current_device(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int ttt_linear_fwd_noalloc(int kind, int qkv_dtype, int B, int H, int N, int d, int b, const void* Q,
                                      const void* K, const void* V, const float* eta, float eta_const,
                                      const float* W0, const float* ln_gamma, const float* ln_beta, float ln_eps,
                                      float* Z, float* W_end, void* hip_stream)
{
    // validation on the host first (the scratch array is never a caller buffer,
    // so it overlaps none)
    const size_t need = ttt_linear_fwd_workspace_bytes(kind, qkv_dtype, B, H, N, d, b);
    if (need > TTT_NOALLOC_SCRATCH_BYTES) return TTT_ERR_WORKSPACE_TOO_SMALL;
    ttt::LinearArgs a;
    int path = TTT_PATH_NONE;
    const int st = check_linear(kind, qkv_dtype, B, H, N, d, b, Q, K, V, eta, eta_const, W0, ln_gamma, ln_beta,
                                ln_eps, Z, W_end, nullptr, 0, a, path, /*internal_workspace=*/true);
    if (st != TTT_OK) return st;
    hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
    hipError_t err;
    if (path == TTT_PATH_SMALL_B) {
        err = ttt::launch_smallb_linear(a, stream);
    } else if (!fast_large(qkv_dtype, d, b, N)) {
        err = ttt::launch_midb_linear_blocks(a, ttt::LC_OUT_DUAL, stream);
    } else {
        void* ptr = nullptr;
        err = scratch_on_current_device(&ptr);
        if (err != hipSuccess) return TTT_ERR_HIP;
        a.workspace = ptr;
        a.workspace_bytes = TTT_NOALLOC_SCRATCH_BYTES;
        err = ttt::launch_large_chunk_linear(a, ttt::LC_OUT_DUAL, stream);
    }
    return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}
