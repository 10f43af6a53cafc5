// mlp_generic.hip -- TTT-MLP forward, f(x) = x + LN(GELU(x W1) W2), for the
// combinations the register-resident kernel (smallb_mlp.hip) does not take:
// chunks of 17..64 tokens at d = 64, and d = 128 (hidden 512) with chunks of
// 1..64 tokens; fp32 or bf16 token streams.
//
// Method: page "How to Master Test-Time Training for Infinite Context LLMs"
// (section "The Math and Architecture of TTT Layers": a small MLP as the inner
// model) in the mini-batch dual form of page "Test-Time Training: Linear
// Complexity Beyond Attention", section "4. Mini-Batch Parallelism (Dual
// Formulation)", per chunk with chunk-start weights W1, W2:
//     A   = K W1,  X2 = GELU(A),  H = X2 W2,
//     G2  = LN backward of 2(K + LN(H) - V),  G1 = (G2 W2^T) * GELU'(A)
//     A_Q = Q W1 - tril(Q K^T) diag(eta) G1,   X2_Q = GELU(A_Q)
//     H_Q = X2_Q W2 - tril(X2_Q X2^T) diag(eta) G2,   Z = Q + LN(H_Q)
//     W1 <- W1 - K^T diag(eta) G1,   W2 <- W2 - X2^T diag(eta) G2
//
// Design: one workgroup of four waves per (sequence, head). At these sizes the
// state does not fit on a compute unit (2 x 256 KB fp32 at d = 128), so it
// lives in memory, as do the chunk's intermediate matrices: the caller's
// workspace holds W1^T, W2^T, X2, X2^T, X2_Q, (eta G1)^T, G2 and (eta G2)^T
// of the unit (about 1.2 MB at d = 128, L2-resident), W2 itself stays in the
// W2_end buffer. Every matrix is stored with the index a product contracts over
// contiguous, so both operands of every MFMA (16x16x32 over features, 16x16x16
// over tokens) are contiguous reads; fp32 operands are split into bf16 terms on
// the fly (two next to bf16 streams, three next to fp32 streams). The chunk's Q
// and K rows and the small matrices (S, S2, H, H_Q) sit in LDS. Phases are
// separated by workgroup barriers with device-scope fences (the intermediates
// written by one wave are read by others).
#include "gelu.h"
#include "kernels.h"
#include "device_common.h"

namespace ttt {
namespace {

constexpr int GT = 256;   // threads: four waves

template <int D, int NG>
struct GenGeom {
    static constexpr int HID = 4 * D;
    static constexpr int BR = 16 * NG;   // rows of a chunk, padded to groups of 16
    // workspace per unit, in floats
    static constexpr size_t W1T = 0;                                  // [HID][D]
    static constexpr size_t W2T = W1T + (size_t)HID * D;              // [D][HID]
    static constexpr size_t X2 = W2T + (size_t)D * HID;               // [BR][HID]
    static constexpr size_t X2T = X2 + (size_t)BR * HID;              // [HID][BR]
    static constexpr size_t X2Q = X2T + (size_t)HID * BR;             // [BR][HID]
    static constexpr size_t G1T = X2Q + (size_t)BR * HID;             // [HID][BR], eta-scaled
    static constexpr size_t D1 = G1T + (size_t)HID * BR;              // [BR][HID], GELU'(A)
    static constexpr size_t G2 = D1 + (size_t)BR * HID;               // [BR][D]
    static constexpr size_t G2T = G2 + (size_t)BR * D;                // [D][BR], eta-scaled
    static constexpr size_t TOTAL = G2T + (size_t)D * BR;
};

template <int D, int NG>
struct alignas(16) GenSmem {
    using G = GenGeom<D, NG>;
    float q[G::BR][D + 4];
    float k[G::BR][D + 4];
    float hm[G::BR][D + 4];        // H, then H_Q
    float sm[G::BR][G::BR + 4];    // tril(S), then tril(S2)
    float eta[G::BR];
};

__device__ __forceinline__ void phase_sync()
{
    __threadfence();
    __syncthreads();
}

// Eight consecutive fp32 values at p as T bf16 terms.
template <int T>
__device__ __forceinline__ void frag8(const float* p, bf16x8 (&out)[T])
{
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    terms8<T>(x, out);
}

template <int T>
__device__ __forceinline__ void frag4(const float* p, bf16x4 (&out)[T])
{
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float x[4] = {a.x, a.y, a.z, a.w};
    terms4<T>(x, out);
}

// acc += A B over k in [0, K) with A row-major [16][lda] (row = lane n) and B
// given as B^T row-major [16][ldb] (column = lane n): 16x16x32 steps.
template <int T>
__device__ __forceinline__ f32x4 mm32(f32x4 acc, const float* A, int lda, const float* Bt, int ldb, int K, int g,
                                      int n)
{
    for (int k0 = 0; k0 < K; k0 += 32) {
        bf16x8 a[T], b[T];
        frag8<T>(A + (size_t)n * lda + k0 + 8 * g, a);
        frag8<T>(Bt + (size_t)n * ldb + k0 + 8 * g, b);
        acc = mma32_terms<T, T>(acc, a, b);
    }
    return acc;
}

// The same over k in steps of 16 (contractions over the tokens of a chunk).
template <int T>
__device__ __forceinline__ f32x4 mm16(f32x4 acc, const float* A, int lda, const float* Bt, int ldb, int K, int g,
                                      int n)
{
    for (int k0 = 0; k0 < K; k0 += 16) {
        bf16x4 a[T], b[T];
        frag4<T>(A + (size_t)n * lda + k0 + 4 * g, a);
        frag4<T>(Bt + (size_t)n * ldb + k0 + 4 * g, b);
        acc = mma16_terms<T, T>(acc, a, b);
    }
    return acc;
}

template <typename S> __device__ __forceinline__ float to_f32(S x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x)
{
    return __builtin_bit_cast(float, (uint32_t)x << 16);
}

// Mean and reciprocal standard deviation of a row of D values (biased
// variance, two passes, eps inside the root).
template <int D>
__device__ __forceinline__ void ln_row(const float* hrow, float eps, float& mu, float& rs)
{
    float s = 0.f;
    for (int j = 0; j < D; ++j) s += hrow[j];
    mu = s * (1.f / D);
    float v = 0.f;
    for (int j = 0; j < D; ++j) {
        const float c = hrow[j] - mu;
        v = fmaf(c, c, v);
    }
    rs = 1.f / sqrtf(v * (1.f / D) + eps);
}

template <int D, int NG, typename S>
__global__ void __launch_bounds__(GT)
mlp_generic_kernel(int H, int N, int b, const S* __restrict__ Qg, const S* __restrict__ Kg,
                   const S* __restrict__ Vg, const float* __restrict__ etag, float eta_const,
                   const float* W1g, const float* W2g,   // may be the W1e / W2e buffers
                   const float* __restrict__ gamma, const float* __restrict__ beta, float eps,
                   float* __restrict__ Zg, float* W1e, float* W2e, float* __restrict__ wsg)
{
    using G = GenGeom<D, NG>;
    constexpr int HID = G::HID, BR = G::BR;
    constexpr int T = sizeof(S) == 2 ? 2 : 3;   // terms of an fp32 operand
    __shared__ GenSmem<D, NG> sm;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
    const size_t unit = blockIdx.x;
    const int h = (int)(unit % H);
    const S* Qu = Qg + unit * (size_t)N * D;
    const S* Ku = Kg + unit * (size_t)N * D;
    const S* Vu = Vg + unit * (size_t)N * D;
    const float* etau = etag ? etag + unit * (size_t)N : nullptr;
    float* Zu = Zg + unit * (size_t)N * D;
    const float* W1u = W1g + unit * (size_t)D * HID;
    const float* W2u = W2g + unit * (size_t)HID * D;
    float* W1o = W1e + unit * (size_t)D * HID;
    float* W2 = W2e + unit * (size_t)HID * D;       // the running W2, [HID][D]
    float* ws = wsg + unit * G::TOTAL;
    float* W1T = ws + G::W1T;
    float* W2T = ws + G::W2T;
    float* X2 = ws + G::X2;
    float* X2T = ws + G::X2T;
    float* X2Q = ws + G::X2Q;
    float* G1T = ws + G::G1T;
    float* D1 = ws + G::D1;
    float* G2 = ws + G::G2;
    float* G2T = ws + G::G2T;
    const float* gam = gamma + h * D;
    const float* bet = beta + h * D;

    // ---- state into place: W1^T, W2 (in W2_end; may be W2_0 itself), W2^T ----
    for (int i = tid; i < D * HID; i += GT) {
        const int r = i / HID, c = i % HID;   // W1[r][c]
        W1T[(size_t)c * D + r] = W1u[i];
        const int hr = i / D, o = i % D;      // W2[hr][o]
        const float v2 = W2u[i];
        W2T[(size_t)o * HID + hr] = v2;
        W2[i] = v2;
    }
    phase_sync();

    const int C = (N + b - 1) / b;
    for (int c = 0; c < C; ++c) {
        const int c0 = c * b, bc = min(b, N - c0);
        // ---- Q, K of the chunk (zero rows past its end), eta ----
        for (int i = tid; i < BR * D; i += GT) {
            const int r = i / D, f = i % D;
            const bool ok = r < bc;
            sm.q[r][f] = ok ? to_f32<S>(Qu[(size_t)(c0 + r) * D + f]) : 0.f;
            sm.k[r][f] = ok ? to_f32<S>(Ku[(size_t)(c0 + r) * D + f]) : 0.f;
        }
        if (tid < BR) sm.eta[tid] = tid < bc ? (etau ? etau[c0 + tid] : eta_const) : 0.f;
        __syncthreads();

        // ---- A = K W1 -> X2 = GELU(A), GELU'(A) ----
        for (int tile = w; tile < NG * (HID / 16); tile += 4) {
            const int rt = tile / (HID / 16), ht = tile % (HID / 16);
            const f32x4 acc = mm32<T>(f32x4{0.f, 0.f, 0.f, 0.f}, &sm.k[16 * rt][0], D + 4,
                                      W1T + (size_t)(16 * ht) * D, D, D, g, n);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + 4 * g + i, hc = 16 * ht + n;
                float x, d1;
                gelu_fd(acc[i], x, d1);
                X2[(size_t)r * HID + hc] = x;
                X2T[(size_t)hc * BR + r] = x;
                D1[(size_t)r * HID + hc] = d1;
            }
        }
        phase_sync();

        // ---- H = X2 W2 ----
        for (int tile = w; tile < NG * (D / 16); tile += 4) {
            const int rt = tile / (D / 16), ot = tile % (D / 16);
            const f32x4 acc = mm32<T>(f32x4{0.f, 0.f, 0.f, 0.f}, X2 + (size_t)(16 * rt) * HID, HID,
                                      W2T + (size_t)(16 * ot) * HID, HID, HID, g, n);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.hm[16 * rt + 4 * g + i][16 * ot + n] = acc[i];
        }
        __syncthreads();

        // ---- G2 = LayerNorm backward of 2 (K + LN(H) - V), one row per thread ----
        if (tid < BR) {
            const int r = tid;
            float mu, rs;
            ln_row<D>(sm.hm[r], eps, mu, rs);
            float u1 = 0.f, u2 = 0.f;
            for (int j = 0; j < D; ++j) {
                const float xh = (sm.hm[r][j] - mu) * rs;
                const float vv = r < bc ? to_f32<S>(Vu[(size_t)(c0 + r) * D + j]) : 0.f;
                const float dx = 2.f * gam[j] * (sm.k[r][j] + gam[j] * xh + bet[j] - vv);
                u1 += dx;
                u2 = fmaf(dx, xh, u2);
            }
            u1 *= 1.f / D;
            u2 *= 1.f / D;
            const float e = sm.eta[r];
            for (int j = 0; j < D; ++j) {
                const float xh = (sm.hm[r][j] - mu) * rs;
                const float vv = r < bc ? to_f32<S>(Vu[(size_t)(c0 + r) * D + j]) : 0.f;
                const float dx = 2.f * gam[j] * (sm.k[r][j] + gam[j] * xh + bet[j] - vv);
                const float g2 = r < bc ? rs * (dx - u1 - xh * u2) : 0.f;
                G2[(size_t)r * D + j] = g2;
                G2T[(size_t)j * BR + r] = e * g2;
            }
        }
        phase_sync();

        // ---- eta G1 = eta (G2 W2^T) * GELU'(A);  tril(S), S = Q K^T ----
        for (int tile = w; tile < NG * (HID / 16); tile += 4) {
            const int rt = tile / (HID / 16), ht = tile % (HID / 16);
            const f32x4 acc = mm32<T>(f32x4{0.f, 0.f, 0.f, 0.f}, G2 + (size_t)(16 * rt) * D, D,
                                      W2 + (size_t)(16 * ht) * D, D, D, g, n);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + 4 * g + i, hc = 16 * ht + n;
                G1T[(size_t)hc * BR + r] = sm.eta[r] * acc[i] * D1[(size_t)r * HID + hc];
            }
        }
        for (int tile = w; tile < NG * NG; tile += 4) {
            const int qt = tile / NG, kt = tile % NG;
            const f32x4 acc = mm32<T>(f32x4{0.f, 0.f, 0.f, 0.f}, &sm.q[16 * qt][0], D + 4, &sm.k[16 * kt][0], D + 4,
                                      D, g, n);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rq = 16 * qt + 4 * g + i, rk = 16 * kt + n;
                sm.sm[rq][rk] = rk <= rq ? acc[i] : 0.f;
            }
        }
        phase_sync();

        // ---- A_Q = Q W1 - tril(S) eta G1 -> X2_Q = GELU(A_Q) ----
        for (int tile = w; tile < NG * (HID / 16); tile += 4) {
            const int rt = tile / (HID / 16), ht = tile % (HID / 16);
            f32x4 acc = mm32<T>(f32x4{0.f, 0.f, 0.f, 0.f}, &sm.q[16 * rt][0], D + 4, W1T + (size_t)(16 * ht) * D, D,
                                D, g, n);
            const f32x4 cz = mm16<T>(f32x4{0.f, 0.f, 0.f, 0.f}, &sm.sm[16 * rt][0], BR + 4,
                                     G1T + (size_t)(16 * ht) * BR, BR, BR, g, n);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                X2Q[(size_t)(16 * rt + 4 * g + i) * HID + 16 * ht + n] = gelu_f(acc[i] - cz[i]);
        }
        phase_sync();

        // ---- tril(S2), S2 = X2_Q X2^T ----
        for (int tile = w; tile < NG * NG; tile += 4) {
            const int qt = tile / NG, kt = tile % NG;
            const f32x4 acc = mm32<T>(f32x4{0.f, 0.f, 0.f, 0.f}, X2Q + (size_t)(16 * qt) * HID, HID,
                                      X2 + (size_t)(16 * kt) * HID, HID, HID, g, n);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rq = 16 * qt + 4 * g + i, rk = 16 * kt + n;
                sm.sm[rq][rk] = rk <= rq ? acc[i] : 0.f;
            }
        }
        __syncthreads();

        // ---- H_Q = X2_Q W2 - tril(S2) eta G2 ----
        for (int tile = w; tile < NG * (D / 16); tile += 4) {
            const int rt = tile / (D / 16), ot = tile % (D / 16);
            f32x4 acc = mm32<T>(f32x4{0.f, 0.f, 0.f, 0.f}, X2Q + (size_t)(16 * rt) * HID, HID,
                                W2T + (size_t)(16 * ot) * HID, HID, HID, g, n);
            const f32x4 cz = mm16<T>(f32x4{0.f, 0.f, 0.f, 0.f}, &sm.sm[16 * rt][0], BR + 4,
                                     G2T + (size_t)(16 * ot) * BR, BR, BR, g, n);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.hm[16 * rt + 4 * g + i][16 * ot + n] = acc[i] - cz[i];
        }
        __syncthreads();

        // ---- Z = Q + LN(H_Q), one row per thread ----
        if (tid < bc) {
            const int r = tid;
            float mu, rs;
            ln_row<D>(sm.hm[r], eps, mu, rs);
            for (int j = 0; j < D; ++j)
                Zu[(size_t)(c0 + r) * D + j] = sm.q[r][j] + gam[j] * ((sm.hm[r][j] - mu) * rs) + bet[j];
        }
        // ---- state updates (every read of this chunk's state is behind the barriers above):
        //      W1^T -= (eta G1)^T K,  W2 -= X2^T (eta G2),  W2^T -= (eta G2)^T X2 ----
        for (int tile = w; tile < (HID / 16) * (D / 16); tile += 4) {
            const int ht = tile / (D / 16), ft = tile % (D / 16);
            // B = K as [feature][token]: gathered from the [token][feature] LDS rows
            f32x4 acc;
            float* dst = W1T + (size_t)(16 * ht) * D + 16 * ft;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = dst[(size_t)(4 * g + i) * D + n];
            for (int k0 = 0; k0 < BR; k0 += 16) {
                bf16x4 a[T], bb[T];
                frag4<T>(G1T + (size_t)(16 * ht + n) * BR + k0 + 4 * g, a);
                float x[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = -sm.k[k0 + 4 * g + j][16 * ft + n];
                terms4<T>(x, bb);
                acc = mma16_terms<T, T>(acc, a, bb);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(size_t)(4 * g + i) * D + n] = acc[i];
        }
        for (int tile = w; tile < (HID / 16) * (D / 16); tile += 4) {
            const int ht = tile / (D / 16), ot = tile % (D / 16);
            float* dst = W2 + (size_t)(16 * ht) * D + 16 * ot;
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = -dst[(size_t)(4 * g + i) * D + n];
            acc = mm16<T>(acc, X2T + (size_t)(16 * ht) * BR, BR, G2T + (size_t)(16 * ot) * BR, BR, BR, g, n);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(size_t)(4 * g + i) * D + n] = -acc[i];
        }
        for (int tile = w; tile < (D / 16) * (HID / 16); tile += 4) {
            const int ot = tile / (HID / 16), ht = tile % (HID / 16);
            float* dst = W2T + (size_t)(16 * ot) * HID + 16 * ht;
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = -dst[(size_t)(4 * g + i) * HID + n];
            acc = mm16<T>(acc, G2T + (size_t)(16 * ot) * BR, BR, X2T + (size_t)(16 * ht) * BR, BR, BR, g, n);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(size_t)(4 * g + i) * HID + n] = -acc[i];
        }
        phase_sync();
    }

    // ---- W1_end from W1^T (W2_end already holds W2) ----
    for (int i = tid; i < D * HID; i += GT) {
        const int r = i / HID, cc = i % HID;
        W1o[i] = W1T[(size_t)cc * D + r];
    }
}

template <int D, int NG, typename S>
hipError_t launch_gen(const MlpArgs& a, float* ws, hipStream_t stream)
{
    hipLaunchKernelGGL((mlp_generic_kernel<D, NG, S>), dim3(a.B * a.H), dim3(GT), 0, stream, a.H, a.N, a.b,
                       static_cast<const S*>(a.Q), static_cast<const S*>(a.K), static_cast<const S*>(a.V), a.eta,
                       a.eta_const, a.W1, a.W2, a.gamma, a.beta, a.eps, a.Z, a.W1_end, a.W2_end, ws);
    return hipGetLastError();
}

template <int D, typename S>
hipError_t launch_d(const MlpArgs& a, float* ws, hipStream_t stream)
{
    const int ng = (a.b + 15) / 16;
    if (ng == 1) return launch_gen<D, 1, S>(a, ws, stream);
    if (ng == 2) return launch_gen<D, 2, S>(a, ws, stream);
    if (ng == 3) return launch_gen<D, 3, S>(a, ws, stream);
    return launch_gen<D, 4, S>(a, ws, stream);
}

template <int D>
size_t per_unit_floats(int b)
{
    const int ng = (b + 15) / 16;
    if (ng == 1) return GenGeom<D, 1>::TOTAL;
    if (ng == 2) return GenGeom<D, 2>::TOTAL;
    if (ng == 3) return GenGeom<D, 3>::TOTAL;
    return GenGeom<D, 4>::TOTAL;
}

}  // namespace

size_t mlp_generic_workspace_bytes(int B, int H, int d, int b)
{
    const size_t per = d == 128 ? per_unit_floats<128>(b) : per_unit_floats<64>(b);
    return (size_t)B * (size_t)H * per * sizeof(float);
}

hipError_t launch_mlp_generic(const MlpArgs& a, void* workspace, hipStream_t stream)
{
    float* ws = static_cast<float*>(workspace);
    if (a.d == 128) return a.dtype == 1 ? launch_d<128, uint16_t>(a, ws, stream) : launch_d<128, float>(a, ws, stream);
    return a.dtype == 1 ? launch_d<64, uint16_t>(a, ws, stream) : launch_d<64, float>(a, ws, stream);
}

}  // namespace ttt
