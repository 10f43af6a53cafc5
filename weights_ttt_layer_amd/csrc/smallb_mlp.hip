// smallb_mlp.hip -- TTT-MLP forward, f(x) = x + LN(GELU(x W1) W2), d = 64,
// hidden = 256, chunks of 1 <= b <= 16 tokens.
//
// Inner model: a small multi-layer perceptron (page "How to Master Test-Time
// Training for Infinite Context LLMs", section "The Math and Architecture of
// TTT Layers"), no biases, GELU in its erf form (erf evaluated with Abramowitz &
// Stegun 7.1.26, |error| <= 1.5e-7), LayerNorm + residual on its output.
// The mini-batch dual form (page "Test-Time Training: Linear Complexity Beyond
// Attention", section "4. Mini-Batch Parallelism (Dual Formulation)") applied
// to both layers, per chunk with chunk-start weights W1, W2:
//     A   = K W1,  X2 = GELU(A),  H = X2 W2,
//     G2  = LN backward of 2(K + LN(H) - V),  G1 = (G2 W2^T) * GELU'(A)
//     A_Q = Q W1 - tril(Q K^T) diag(eta) G1,   X2_Q = GELU(A_Q)
//     H_Q = X2_Q W2 - tril(X2_Q X2^T) diag(eta) G2,   Z = Q + LN(H_Q)
//     W1 <- W1 - K^T diag(eta) G1,   W2 <- W2 - X2^T diag(eta) G2
//
// Design (gfx950): one workgroup of four waves per (sequence, head). The state
// stays in MFMA accumulators for the whole scan: wave w holds W1 columns
// [64w, 64w+64), W2 columns [16w, 16w+16) and, for the backward product
// G2 W2^T, a second copy W2^T with columns [64w, 64w+64) that receives the
// same update (K W1 and X2 W2 contract over the state's rows and read the
// accumulators directly; G2 W2^T contracts over W2's columns, which is the row
// index of W2^T). Activations that a product needs in another orientation
// (X2, X2_Q, G2) go through row-padded fp32 LDS tiles. fp32 operands are split
// into bf16 terms as in the linear kernel.
#include "kernels.h"
#include "smallb_common.h"

namespace ttt {
namespace {

using namespace smallb;

constexpr int HID = 256;
constexpr int XS = HID + 4;     // row stride of [token][hidden] fp32 tiles
constexpr int GS = D + 4;       // row stride of [token][d] fp32 tiles
constexpr int XTS = ROWS + 4;   // row stride of the [hidden][token] fp32 tile
constexpr int XB = HID + 8;     // row stride of [token][hidden] bf16 term tiles

// terms of an fp32 operand next to token streams of type S
template <typename S>
constexpr int fp_terms() { return Stor<S>::TERMS == 1 ? 2 : 3; }

// GELU(A) and GELU(A_Q) are written once, already split into their bf16
// operand terms, by the wave that owns the hidden slice; the products over the
// hidden dimension then read ready terms instead of every wave splitting every
// row again.
template <typename S>
struct alignas(16) MlpSmem {
    Stage<S> st[2];
    uint16_t x2b[fp_terms<S>()][ROWS * XB];    // GELU(K W1) terms, [token][hidden]
    float x2t[HID * XTS];                      // GELU(K W1), [hidden][token]
    uint16_t x2qb[fp_terms<S>()][ROWS * XB];   // GELU(A_Q) terms, [token][hidden]
    float d1[ROWS * XS];                       // GELU'(A), [token][hidden]
    float g2[ROWS * GS];     // dl/dH at the chunk-start weights (no eta), [token][d]
    float red[3][4][ROWS][2];
    float w2mean[HID];       // row means of W2_0 (removed from the carried state)
};

// GELU(a) = a Phi(a), Phi(a) = (1 + erf(a / sqrt 2)) / 2, and its derivative
// Phi(a) + a phi(a). erf comes from Abramowitz & Stegun, "Handbook of
// Mathematical Functions", formula 7.1.26: for x >= 0,
//     erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
//     t = 1 / (1 + p x),   |error| <= 1.5e-7,
// extended to x < 0 by odd symmetry. Only Phi = (1 + erf) / 2 is used, so the
// absolute error bound is the one that matters. exp(-x^2) = exp(-a^2 / 2) is
// also the Gaussian factor of phi, shared by the derivative.
constexpr float AS_P = 0.3275911f;
constexpr float AS_A1 = 0.254829592f, AS_A2 = -0.284496736f, AS_A3 = 1.421413741f,
                AS_A4 = -1.453152027f, AS_A5 = 1.061405429f;

__device__ __forceinline__ float phi_cdf(float a, float& gauss)
{
    const float x = fabsf(a) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(AS_P, x, 1.f));
    gauss = __expf(-x * x);
    const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, AS_A5, AS_A4), AS_A3), AS_A2), AS_A1);
    const float erfx = 1.f - poly * gauss;
    return 0.5f * (1.f + copysignf(erfx, a));
}

__device__ __forceinline__ float gelu_f(float a)
{
    float gauss;
    return a * phi_cdf(a, gauss);
}

// GELU(a) and d/da GELU(a) = Phi(a) + a exp(-a^2/2) / sqrt(2 pi)
__device__ __forceinline__ void gelu_fd(float a, float& f, float& fd)
{
    float gauss;
    const float c = phi_cdf(a, gauss);
    f = a * c;
    fd = fmaf(a * 0.39894228040143267794f, gauss, c);
}

// Operand fragment of a pre-split [token][hidden] tile: per term, four entries
// at row + o and four at row + o + 16 (the k order of load_a8).
template <int T>
__device__ __forceinline__ void load_terms8(const uint16_t (*tile)[ROWS * XB], int off, bf16x8 (&out)[T])
{
#pragma unroll
    for (int s = 0; s < T; ++s) {
        const uint2 a = *reinterpret_cast<const uint2*>(tile[s] + off);
        const uint2 b = *reinterpret_cast<const uint2*>(tile[s] + off + 16);
        out[s] = __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
    }
}

// Split v into T bf16 terms and store them at tile[s][off].
template <int T>
__device__ __forceinline__ void store_terms(uint16_t (*tile)[ROWS * XB], int off, float v)
{
    __bf16 t[T];
    split_terms<T>(v, t);
#pragma unroll
    for (int s = 0; s < T; ++s) tile[s][off] = __builtin_bit_cast(uint16_t, t[s]);
}

template <typename S>
__device__ __forceinline__ void mlp_chunk(const Stage<S>& st, MlpSmem<S>& sm, f32x4 (&W1acc)[4][4],
                                          f32x4 (&W2acc)[16], f32x4 (&W2Tacc)[4][4], int c0, int bc,
                                          float gam, float bet, float eps, float* __restrict__ Zu,
                                          int w, int g, int n)
{
    constexpr int TIN = Stor<S>::TERMS;
    constexpr int TS = (TIN == 1) ? 2 : 3;
    constexpr int STRIDE = Stor<S>::STRIDE;
    const int col = 16 * w + n;

    // ---- (1) A = K W1 and Q W1 for this wave's four hidden tiles ----
    f32x4 ak[4], aq[4];
    {
        bf16x8 ka[2][TIN], qa[2][TIN];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int o0 = n * STRIDE + 32 * p + 4 * g;
            load_a8<S, TIN>(st.k + o0, st.k + o0 + 16, ka[p]);
            load_a8<S, TIN>(st.q + o0, st.q + o0 + 16, qa[p]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            ak[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            aq[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                bf16x8 wb[TS];
                b8_from_acc<TS>(W1acc[2 * p][t], W1acc[2 * p + 1][t], wb);
                ak[t] = mma32_terms<TIN, TS>(ak[t], ka[p], wb);
                aq[t] = mma32_terms<TIN, TS>(aq[t], qa[p], wb);
            }
        }
    }
    // ---- (2) S^T = K Q^T: lane (g, n) holds S[n][4g+i] = q_n . k_{4g+i} ----
    f32x4 sT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        bf16x8 ka[TIN], qb[TIN];
        const int o = n * STRIDE + 32 * p + 8 * g;
        load_a8<S, TIN>(st.k + o, st.k + o + 4, ka);
        load_a8<S, TIN>(st.q + o, st.q + o + 4, qb);
        sT = mma32_terms<TIN, TIN>(sT, ka, qb);
    }
    float et[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) et[i] = st.eta[4 * g + i];

    // ---- (3) X2 = GELU(A), GELU'(A); publish X2 in both orientations ----
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x2, d1;
            gelu_fd(ak[t][i], x2, d1);
            const int hcol = 64 * w + 16 * t + n;
            store_terms<TS>(sm.x2b, (4 * g + i) * XB + hcol, x2);
            sm.x2t[hcol * XTS + 4 * g + i] = x2;
            sm.d1[(4 * g + i) * XS + hcol] = d1;
        }
    __syncthreads();

    // ---- (4) H = X2 W2 for columns [16w, 16w+16) ----
    f32x4 hk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        bf16x8 xa[TS], wb[TS];
        load_terms8<TS>(sm.x2b, n * XB + 32 * p + 4 * g, xa);
        b8_from_acc<TS>(W2acc[2 * p], W2acc[2 * p + 1], wb);
        hk = mma32_terms<TS, TS>(hk, xa, wb);
    }

    // ---- (5) LayerNorm forward and backward: G2 = dl/dH ----
    float g2[4];
    {
        float s1[4], s2[4], mu[4], rs[4], xh[4], dxh[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s1[i] = hk[i];
            s2[i] = hk[i] * hk[i];
        }
        xwave_row_sums(s1, s2, sm.red[0], w, g, n);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mu[i] = s1[i] * (1.f / D);
            const float var = fmaxf(s2[i] * (1.f / D) - mu[i] * mu[i], 0.f);
            rs[i] = 1.f / sqrtf(var + eps);
            xh[i] = (hk[i] - mu[i]) * rs[i];
            const float kk = Stor<S>::f(st.k[(4 * g + i) * STRIDE + col]);
            const float vv = Stor<S>::f(st.v[(4 * g + i) * STRIDE + col]);
            dxh[i] = 2.f * (kk + gam * xh[i] + bet - vv) * gam;
            s1[i] = dxh[i];
            s2[i] = dxh[i] * xh[i];
        }
        xwave_row_sums(s1, s2, sm.red[1], w, g, n);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            g2[i] = rs[i] * (dxh[i] - s1[i] * (1.f / D) - xh[i] * (s2[i] * (1.f / D)));
            if (4 * g + i >= bc) g2[i] = 0.f;
            sm.g2[(4 * g + i) * GS + col] = g2[i];
        }
    }
    __syncthreads();

    // ---- (6) G1 = (G2 W2^T) * GELU'(A) for this wave's hidden tiles ----
    bf16x8 g2a[2][TS];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const float* r0 = sm.g2 + n * GS + 32 * p + 4 * g;
        load_a8<float, TS>(r0, r0 + 16, g2a[p]);
    }
    bf16x4 gb1[4][TS];   // -diag(eta) G1, B operand (k = token)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            bf16x8 wb[TS];
            b8_from_acc<TS>(W2Tacc[2 * p][t], W2Tacc[2 * p + 1][t], wb);
            acc = mma32_terms<TS, TS>(acc, g2a[p], wb);
        }
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            x[i] = (4 * g + i < bc) ? -et[i] * acc[i] * sm.d1[(4 * g + i) * XS + 64 * w + 16 * t + n] : 0.f;
        terms4<TS>(x, gb1[t]);
    }

    // ---- (7) A_Q = Q W1 - tril(S) diag(eta) G1; X2_Q = GELU(A_Q) ----
    bf16x4 sa[TS];
    {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (4 * g + i <= n) ? sT[i] : 0.f;
        terms4<TS>(x, sa);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        aq[t] = mma16_terms<TS, TS>(aq[t], sa, gb1[t]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            store_terms<TS>(sm.x2qb, (4 * g + i) * XB + 64 * w + 16 * t + n, gelu_f(aq[t][i]));
    }
    // W1 -= K^T diag(eta) G1 now (A_Q used W1_c above), so the G1 terms die here.
    // A = K^T tile r: row = feature 16r+n, k = token.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = Stor<S>::f(st.k[(4 * g + j) * STRIDE + 16 * r + n]);
        bf16x4 kt[TIN];
        terms4<TIN>(x, kt);
#pragma unroll
        for (int t = 0; t < 4; ++t) W1acc[r][t] = mma16_terms<TIN, TS>(W1acc[r][t], kt, gb1[t]);
    }
    __syncthreads();

    // ---- (8) S2^T = X2 X2_Q^T: lane (g, n) holds S2[n][4g+i] ----
    f32x4 s2T = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        bf16x8 xa[TS], xq[TS];
        load_terms8<TS>(sm.x2b, n * XB + 32 * p + 4 * g, xa);
        load_terms8<TS>(sm.x2qb, n * XB + 32 * p + 4 * g, xq);
        s2T = mma32_terms<TS, TS>(s2T, xa, xq);
    }
    // -diag(eta) G2 as B operand
    bf16x4 gb2[TS];
    {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = -et[i] * g2[i];
        terms4<TS>(x, gb2);
    }

    // ---- (9) H_Q = X2_Q W2 - tril(S2) diag(eta) G2 ----
    f32x4 hq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        bf16x8 xq[TS], wb[TS];
        load_terms8<TS>(sm.x2qb, n * XB + 32 * p + 4 * g, xq);
        b8_from_acc<TS>(W2acc[2 * p], W2acc[2 * p + 1], wb);
        hq = mma32_terms<TS, TS>(hq, xq, wb);
    }
    {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (4 * g + i <= n) ? s2T[i] : 0.f;
        bf16x4 s2a[TS];
        terms4<TS>(x, s2a);
        hq = mma16_terms<TS, TS>(hq, s2a, gb2);
    }

    // ---- (10) Z = Q + LN(H_Q) ----
    {
        float s1[4], s2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s1[i] = hq[i];
            s2[i] = hq[i] * hq[i];
        }
        xwave_row_sums(s1, s2, sm.red[2], w, g, n);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mu = s1[i] * (1.f / D);
            const float var = fmaxf(s2[i] * (1.f / D) - mu * mu, 0.f);
            const float rs = 1.f / sqrtf(var + eps);
            const float qq = Stor<S>::f(st.q[(4 * g + i) * STRIDE + col]);
            const float z = qq + gam * ((hq[i] - mu) * rs) + bet;
            if (4 * g + i < bc) Zu[(size_t)(c0 + 4 * g + i) * D + col] = z;
        }
    }

    // ---- (11) state updates ----
    // W2 -= X2^T diag(eta) G2   (A = X2^T tile r: row = hidden 16r+n, k = token)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float4 v = *reinterpret_cast<const float4*>(sm.x2t + (16 * r + n) * XTS + 4 * g);
        float x[4] = {v.x, v.y, v.z, v.w};
        bf16x4 xa[TS];
        terms4<TS>(x, xa);
        W2acc[r] = mma16_terms<TS, TS>(W2acc[r], xa, gb2);
    }
    // W2^T -= diag(eta)-scaled G2^T X2   (A = G2^T tile r: row = feature 16r+n, k = token)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = et[j] * sm.g2[(4 * g + j) * GS + 16 * r + n];
        bf16x4 ga[TS];
        terms4<TS>(x, ga);
        (void)x;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            // terms of -X2 (the split of a negated value is the negated split)
            bf16x4 xb[TS];
#pragma unroll
            for (int sT = 0; sT < TS; ++sT) {
                uint32_t u[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    u[i] = (uint32_t)sm.x2b[sT][(4 * g + i) * XB + 64 * w + 16 * t + n] ^ 0x8000u;
                xb[sT] = __builtin_bit_cast(bf16x4, make_uint2(u[0] | (u[1] << 16), u[2] | (u[3] << 16)));
            }
            W2Tacc[r][t] = mma16_terms<TS, TS>(W2Tacc[r][t], ga, xb);
        }
    }
}

template <typename S>
__global__ void __launch_bounds__(THREADS)
smallb_mlp_kernel(int H, int N, int b, const S* __restrict__ Qg, const S* __restrict__ Kg,
                  const S* __restrict__ Vg, const float* __restrict__ etag, float eta_const,
                  const float* __restrict__ W1g, const float* __restrict__ W2g,
                  const float* __restrict__ gamma, const float* __restrict__ beta, float eps,
                  float* __restrict__ Zg, float* __restrict__ W1e, float* __restrict__ W2e)
{
    constexpr int PPT = (Pieces<S>::TOTAL + THREADS - 1) / THREADS;
    __shared__ MlpSmem<S> sm;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int n = lane & 15;

    const size_t unit = blockIdx.x;
    const int h = (int)(unit % H);
    const S* Qu = Qg + unit * (size_t)N * D;
    const S* Ku = Kg + unit * (size_t)N * D;
    const S* Vu = Vg + unit * (size_t)N * D;
    const float* etau = etag ? etag + unit * (size_t)N : nullptr;
    float* Zu = Zg + unit * (size_t)N * D;
    const float* W1u = W1g + unit * (size_t)D * HID;
    const float* W2u = W2g + unit * (size_t)HID * D;

    f32x4 W1acc[4][4], W2acc[16], W2Tacc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                W1acc[r][t][i] = W1u[(16 * r + 4 * g + i) * HID + 64 * w + 16 * t + n];
                W2Tacc[r][t][i] = W2u[(64 * w + 16 * t + n) * D + 16 * r + 4 * g + i];
            }
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) W2acc[r][i] = W2u[(16 * r + 4 * g + i) * D + 16 * w + n];
    const float gam = gamma[h * D + 16 * w + n];
    const float bet = beta[h * D + 16 * w + n];

    // W2 is carried with each row's mean over the output features removed.
    // LayerNorm ignores a constant added to a whole row of H = X2 W2, and its
    // gradient G2 sums to zero over the features, so neither the update
    // X2^T Gt2 nor the product G2 W2^T sees the means, and they never change;
    // they are added back to W2_end. Rows of H then have a near-zero mean
    // whatever W2_0 holds, so the one-pass variance keeps its precision.
    // Wave w holds hidden rows 64w + 16t + n of W2^T in full (columns 16r + 4g + i).
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) s += (W2Tacc[r][t][0] + W2Tacc[r][t][1]) + (W2Tacc[r][t][2] + W2Tacc[r][t][3]);
        s = xrow4_sum(s) * (1.f / D);
        if (g == 0) sm.w2mean[64 * w + 16 * t + n] = s;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) W2Tacc[r][t][i] -= s;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) W2acc[r][i] -= sm.w2mean[16 * r + 4 * g + i];

    const int nchunks = (N + b - 1) / b;
    // one chunk in flight: loaded during the previous chunk's (long) body
    uint4 pf[PPT];
    float pe = 0.f;
    load_chunk<S, PPT>(pf, pe, 0, b, N, tid, Qu, Ku, Vu, etau, eta_const);
    for (int c = 0; c < nchunks; ++c) {
        const int c0 = c * b;
        const int bc = min(b, N - c0);
        store_chunk<S, PPT>(sm.st[c & 1], pf, pe, tid, bc);
        if (c + 1 < nchunks) load_chunk<S, PPT>(pf, pe, c + 1, b, N, tid, Qu, Ku, Vu, etau, eta_const);
        __syncthreads();
        mlp_chunk<S>(sm.st[c & 1], sm, W1acc, W2acc, W2Tacc, c0, bc, gam, bet, eps, Zu, w, g, n);
    }

    float* W1o = W1e + unit * (size_t)D * HID;
    float* W2o = W2e + unit * (size_t)HID * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                W1o[(16 * r + 4 * g + i) * HID + 64 * w + 16 * t + n] = W1acc[r][t][i];
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i)   // the row means added back (one rounding)
            W2o[(16 * r + 4 * g + i) * D + 16 * w + n] = W2acc[r][i] + sm.w2mean[16 * r + 4 * g + i];
}

template <typename S>
hipError_t launch_typed(const MlpArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((smallb_mlp_kernel<S>), dim3(a.B * a.H), dim3(THREADS), 0, stream, a.H, a.N,
                       a.b, static_cast<const S*>(a.Q), static_cast<const S*>(a.K),
                       static_cast<const S*>(a.V), a.eta, a.eta_const, a.W1, a.W2, a.gamma, a.beta,
                       a.eps, a.Z, a.W1_end, a.W2_end);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_smallb_mlp(const MlpArgs& a, hipStream_t stream)
{
    return a.dtype == 1 ? launch_typed<uint16_t>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace ttt
