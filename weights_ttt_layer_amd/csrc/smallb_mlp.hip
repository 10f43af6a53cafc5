// smallb_mlp.hip -- TTT-MLP forward, f(x) = x + LN(GELU(x W1) W2), d = 64,
// hidden = 256, chunks of 1 <= b <= 16 tokens, bf16 or fp32 token streams.
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
// Design (gfx950): one workgroup of four waves per (sequence, head); wave w
// owns the hidden slice h in [64w, 64w + 64) of both layers and keeps, for the
// whole scan, in fp32 MFMA accumulator tiles:
//     W1[:, slice]    rows = input features, columns = hidden
//     W2[slice, :]    rows = hidden, columns = output features
//     W2[slice, :]^T  rows = output features, columns = hidden (for G2 W2^T)
// Every product is taken in the orientation in which its operands are ready:
//  * A^T = W1^T K^T and A_Q^T (the W1 tiles as A operand) leave one token per
//    lane; GELU, GELU' and the eta scaling act there in registers.
//  * H^T = W2^T X2^T takes the W2 tiles as A operand and X2^T straight from the
//    registers as B operand (the C layout of a transposed product is the B
//    operand of the next one, up to a fixed permutation of k); its four
//    slice-partials meet in LDS. Wave w sums them for tokens 4w .. 4w + 3 only,
//    one token per DPP row of 16 lanes (four features a lane), runs the
//    LayerNorm forward and backward there and writes G2 and the -eta G2 terms
//    to LDS; after a barrier every wave reads G2 back in its own layout.
//  * G1^T = (W2 G2^T) * GELU'(A)^T and the output-side H_Q^T, S2^T = X2 X2_Q^T
//    likewise; S2^T's slice-partials meet in LDS with H_Q^T's. Wave w completes
//    H_Q^T tile w (output features 16w .. 16w + 15) and its part of the output
//    LayerNorm sums; the four parts meet in LDS behind a barrier.
//  * Products over tokens (the causal terms and the state updates) need the
//    token index along k: -Gt1 and X2 are written as bf16 terms to wave-private
//    [token][feature] LDS tiles, -Gt2 to one shared tile, and read back with
//    the transpose read ds_read_b64_tr_b16.
// Four workgroup barriers per chunk (the H partials, G2, the H_Q/S2 partials,
// the output LayerNorm sums); the next chunk is staged into the other LDS
// buffer after the first.
//
// W2 is carried with each row's mean over the output features removed (a row
// of W2 belongs to one wave, so the means are wave-local): LayerNorm ignores a
// constant added to a whole row of H, and G2 sums to zero over the features, so
// neither G2 W2^T nor the update sees the means and they never change. Rows of
// H then have a near-zero mean whatever W2_0 holds, so the one-pass variance
// keeps its precision. W2_end = W2_0 + (accumulated change), bit for bit W2_0
// when nothing moved.
//
// Precision: fp32 operands (state, activations, gradients, scores) as two bf16
// terms next to bf16 streams, three next to fp32 streams; fp32 accumulation.
#include "gelu.h"
#include "kernels.h"
#include "smallb_common.h"

namespace ttt {
namespace {

using namespace smallb;

constexpr int HID = 256;

// [16 token][64 column] bf16 tiles with 128-byte rows; the 16-byte piece p of
// row r sits at slot p ^ (r & 7), which keeps both the 8-byte row writes and
// the transpose reads of four rows free of bank conflicts.
__device__ __forceinline__ int toff(int r, int col)
{
    return r * 128 + (((col >> 3) ^ (r & 7)) << 4) + (col & 7) * 2;
}

// Transpose read: lane (g, n) receives column col0 + n of rows 4g .. 4g + 3
// (called with row = 4g + n/4, col = col0 + 4(n%4)).
__device__ __forceinline__ bf16x4 tr4(const uint16_t* tile, int row, int col)
{
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_bf16x4*)(reinterpret_cast<const char*>(tile) + toff(row, col)));
}

// Four values of one token (columns col .. col + 3) as T bf16 terms, also
// written to the term tiles at row `r`.
template <int T>
__device__ __forceinline__ void put4(uint16_t (*tile)[16 * 64], int r, int col, const float (&x)[4], bf16x4 (&t)[T])
{
    terms4<T>(x, t);
#pragma unroll
    for (int s = 0; s < T; ++s)
        *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(tile[s]) + toff(r, col)) = t[s];
}

__device__ __forceinline__ bf16x8 cat8(const bf16x4& a, const bf16x4& b)
{
    const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
    return __builtin_bit_cast(bf16x8, make_uint4(ua.x, ua.y, ub.x, ub.y));
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename S, int TS>
struct alignas(16) MlpSmem {
    Stage<S> st[2];
    float4 hp[4][4][64];            // H^T slice-partials [wave][output tile][lane]
    float4 hqp[4][4][64];           // H_Q^T slice-partials
    float4 s2p[4][64];              // S2^T slice-partials
    uint16_t x2t[4][TS][16 * 64];   // per wave: X2 terms, [token][hidden of the slice]
    uint16_t g1t[4][TS][16 * 64];   // per wave: -Gt1 terms, [token][hidden of the slice]
    uint16_t g2t[TS][16 * 64];      // -Gt2 terms, [token][output feature]
    float4 g2s[16][16];             // G2 (fp32), [token][output features 4j .. 4j + 3]
    float2 xs[16][4];               // output LayerNorm partial sums [token][wave]
    float w2m[4][64];               // row means of W2_0 over the output features
    float4 gb[2][4][4];             // LayerNorm gamma, beta: [which][output tile][g]
};

template <typename S>
__global__ void __launch_bounds__(THREADS)
smallb_mlp_kernel(int H, int N, int b, const S* __restrict__ Qg, const S* __restrict__ Kg,
                  const S* __restrict__ Vg, const float* __restrict__ etag, float eta_const,
                  const float* __restrict__ W1g, const float* __restrict__ W2g,
                  const float* __restrict__ gamma, const float* __restrict__ beta, float eps,
                  float* __restrict__ Zg, float* __restrict__ W1e, float* __restrict__ W2e)
{
    constexpr int TIN = Stor<S>::TERMS;
    constexpr int TS = (TIN == 1) ? 2 : 3;
    constexpr int STRIDE = Stor<S>::STRIDE;
    constexpr int PPT = (Pieces<S>::TOTAL + THREADS - 1) / THREADS;
    __shared__ MlpSmem<S, TS> sm;

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
    const int hs = 64 * w;   // first hidden index of this wave's slice

    // ---- resident state ----
    f32x4 W1[4][4];    // W1[r][t][i]  = W1[16r + 4g + i][hs + 16t + n]
    f32x4 W2[4][4];    // W2[a][o][i]  = W2[hs + 16a + 4g + i][16o + n]
    f32x4 W2T[4][4];   // W2T[r][t][i] = W2[hs + 16t + n][16r + 4g + i]
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                W1[r][t][i] = W1u[(16 * r + 4 * g + i) * HID + hs + 16 * t + n];
                W2[r][t][i] = W2u[(hs + 16 * r + 4 * g + i) * D + 16 * t + n];
                W2T[r][t][i] = W2u[(hs + 16 * t + n) * D + 16 * r + 4 * g + i];
            }
    // W2's row means (hidden rows of this wave's slice), removed from both copies
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s = row16_sum((W2[a][0][i] + W2[a][1][i]) + (W2[a][2][i] + W2[a][3][i]));
            if (n == 0) sm.w2m[w][16 * a + 4 * g + i] = s * (1.f / D);
        }
    wave_lds_sync();
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float m = sm.w2m[w][16 * a + 4 * g + i];
#pragma unroll
            for (int o = 0; o < 4; ++o) W2[a][o][i] -= m;
        }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float m = sm.w2m[w][16 * t + n];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) W2T[r][t][i] -= m;
    }

    // LayerNorm parameters, read from LDS where used: gb[0][o][g] holds gamma of
    // output features 16o + 4g .. 16o + 4g + 3, gb[1] beta
    if (tid < 32) {
        const int which = tid >> 4, o = (tid >> 2) & 3, gg = tid & 3;
        const float* src = (which ? beta : gamma) + h * D + 16 * o + 4 * gg;
        sm.gb[which][o][gg] = make_float4(src[0], src[1], src[2], src[3]);
    }

    const int nchunks = (N + b - 1) / b;
    uint4 pf[PPT];
    float pe = 0.f;
    load_chunk<S, PPT>(pf, pe, 0, b, N, tid, Qu, Ku, Vu, etau, eta_const);
    store_chunk<S, PPT>(sm.st[0], pf, pe, tid, min(b, N));
    if (nchunks > 1) load_chunk<S, PPT>(pf, pe, 1, b, N, tid, Qu, Ku, Vu, etau, eta_const);
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const Stage<S>& st = sm.st[c & 1];
        const int bc = min(b, N - c * b);

        // ================= phase 1: first layer, H^T partial =================
        // K and Q rows of token n as operands over the input features (permuted k)
        bf16x8 ka[2][TIN], qa[2][TIN];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int o0 = n * STRIDE + 32 * p + 4 * g;
            load_a8<S, TIN>(st.k + o0, st.k + o0 + 16, ka[p]);
            load_a8<S, TIN>(st.q + o0, st.q + o0 + 16, qa[p]);
        }
        // A^T, A_Q0^T: lane (g, n) = token n, hidden hs + 16t + 4g + i
        f32x4 aT[4], aqT[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            aT[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            aqT[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                bf16x8 wb[TS];
                b8_from_acc<TS>(W1[2 * p][t], W1[2 * p + 1][t], wb);
                aT[t] = mma32_terms<TS, TIN>(aT[t], wb, ka[p]);
                aqT[t] = mma32_terms<TS, TIN>(aqT[t], wb, qa[p]);
            }
        }
        // X2 = GELU(A) and GELU'(A); X2 terms to the LDS tile (for the W2 updates)
        // and, in registers, as the k = hidden operand of H^T and S2^T
        float d1[4][4];
        bf16x4 x2q4[4][TS];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) gelu_fd(aT[t][i], x[i], d1[t][i]);
            put4<TS>(sm.x2t[w], n, 16 * t + 4 * g, x, x2q4[t]);
        }
        bf16x8 x2b[2][TS];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int s = 0; s < TS; ++s) x2b[p][s] = cat8(x2q4[2 * p][s], x2q4[2 * p + 1][s]);
        // H^T slice-partial (the W2 tiles as A operand: row = output feature, k =
        // hidden): lane = token n, output features 16o + 4g + i
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                bf16x8 wb[TS];
                b8_from_acc<TS>(W2[2 * p][o], W2[2 * p + 1][o], wb);
                acc = mma32_terms<TS, TS>(acc, wb, x2b[p]);
            }
            sm.hp[w][o][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
        __syncthreads();

        // ================= phase 2: LayerNorm gradient, G1, the query side =================
        // the next chunk into the other buffer (its last reader finished before the barrier)
        if (c + 1 < nchunks) {
            store_chunk<S, PPT>(sm.st[(c + 1) & 1], pf, pe, tid, min(b, N - (c + 1) * b));
            if (c + 2 < nchunks) load_chunk<S, PPT>(pf, pe, c + 2, b, N, tid, Qu, Ku, Vu, etau, eta_const);
        }
        const float eta_n = st.eta[n];
        // LayerNorm forward / backward of H, four tokens per wave: lane l takes
        // token tk = 4w + l / 16 and output features f0 .. f0 + 3 (f0 = 4 (l % 16)),
        // so the 16 lanes of a DPP row hold one token's 64 features. G2 and the
        // -eta G2 terms go to LDS, from where every wave takes G2 in its layout.
        {
            const int tk = 4 * w + (lane >> 4), f0 = 4 * (lane & 15);
            const int o = f0 >> 4, gq = (f0 >> 2) & 3;
            float4 hs = sm.hp[0][o][16 * gq + tk];
#pragma unroll
            for (int ww = 1; ww < 4; ++ww) {
                const float4 u = sm.hp[ww][o][16 * gq + tk];
                hs = make_float4(hs.x + u.x, hs.y + u.y, hs.z + u.z, hs.w + u.w);
            }
            const float hv[4] = {hs.x, hs.y, hs.z, hs.w};
            float s1 = (hv[0] + hv[1]) + (hv[2] + hv[3]);
            float s2 = fmaf(hv[0], hv[0], hv[1] * hv[1]) + fmaf(hv[2], hv[2], hv[3] * hv[3]);
            s1 = row16_sum(s1);
            s2 = row16_sum(s2);
            const float mu = s1 * (1.f / D);
            const float rs = __builtin_amdgcn_rsqf(fmaxf(s2 * (1.f / D) - mu * mu, 0.f) + eps);
            const float4 kk = load4_f32<S>(st.k + tk * STRIDE + f0);
            const float4 vv = load4_f32<S>(st.v + tk * STRIDE + f0);
            const float4 ga = sm.gb[0][o][gq], be = sm.gb[1][o][gq];
            const float kv[4] = {kk.x - vv.x, kk.y - vv.y, kk.z - vv.z, kk.w - vv.w};
            const float gam[4] = {ga.x, ga.y, ga.z, ga.w}, bet[4] = {be.x, be.y, be.z, be.w};
            float xh[4], dx[4], u1 = 0.f, u2 = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xh[i] = (hv[i] - mu) * rs;
                dx[i] = 2.f * gam[i] * (kv[i] + gam[i] * xh[i] + bet[i]);
                u1 += dx[i];
                u2 = fmaf(dx[i], xh[i], u2);
            }
            u1 = row16_sum(u1);
            u2 = row16_sum(u2);
            const float m1 = u1 * (1.f / D), m2 = u2 * (1.f / D);
            float gv[4], y[4];
            const float et = st.eta[tk];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gv[i] = (tk < bc) ? rs * (dx[i] - m1 - xh[i] * m2) : 0.f;
                y[i] = -et * gv[i];
            }
            sm.g2s[tk][f0 >> 2] = make_float4(gv[0], gv[1], gv[2], gv[3]);
            bf16x4 tmp[TS];
            put4<TS>(sm.g2t, tk, f0, y, tmp);
        }
        __syncthreads();
        // G2^T as the k = output-feature operand (lane (g, n): token n, features 16o + 4g + i)
        bf16x8 g2b[2][TS];
        {
            bf16x4 q4[4][TS];
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                const float4 v = sm.g2s[n][4 * o + g];
                const float x[4] = {v.x, v.y, v.z, v.w};
                terms4<TS>(x, q4[o]);
            }
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int s = 0; s < TS; ++s) g2b[p][s] = cat8(q4[2 * p][s], q4[2 * p + 1][s]);
        }
        // -Gt1^T = -eta (W2 G2^T) * GELU'(A)^T; its terms to this wave's tile
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                bf16x8 wt[TS];
                b8_from_acc<TS>(W2T[2 * p][t], W2T[2 * p + 1][t], wt);
                acc = mma32_terms<TS, TS>(acc, wt, g2b[p]);
            }
            const float x[4] = {-eta_n * acc[0] * d1[t][0], -eta_n * acc[1] * d1[t][1], -eta_n * acc[2] * d1[t][2],
                                -eta_n * acc[3] * d1[t][3]};
            bf16x4 tmp[TS];
            put4<TS>(sm.g1t[w], n, 16 * t + 4 * g, x, tmp);
        }
        wave_lds_sync();
        // -Gt1[token 4g + j][hidden hs + 16t + n]: A operand of the causal term, B of the W1 update
        bf16x4 g1n[4][TS];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int s = 0; s < TS; ++s) g1n[t][s] = tr4(sm.g1t[w][s], 4 * g + (n >> 2), 16 * t + 4 * (n & 3));
        // tril(S)^T, S^T = K Q^T: lane (g, n) holds S[query n][key 4g + i]
        bf16x4 sb[TS];
        {
            f32x4 sT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                bf16x8 kn[TIN], qn[TIN];
                const int o = n * STRIDE + 32 * p + 8 * g;
                load_a8<S, TIN>(st.k + o, st.k + o + 4, kn);
                load_a8<S, TIN>(st.q + o, st.q + o + 4, qn);
                sT = mma32_terms<TIN, TIN>(sT, kn, qn);
            }
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (4 * g + i <= n) ? sT[i] : 0.f;
            terms4<TS>(x, sb);
        }
        // A_Q^T = A_Q0^T - Gt1^T tril(S)^T; X2_Q = GELU(A_Q), as the k = hidden operand
        bf16x8 x2qb[2][TS];
        {
            bf16x4 q4[4][TS];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                aqT[t] = mma16_terms<TS, TS>(aqT[t], g1n[t], sb);
                float x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = gelu_f(aqT[t][i]);
                terms4<TS>(x, q4[t]);
            }
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int s = 0; s < TS; ++s) x2qb[p][s] = cat8(q4[2 * p][s], q4[2 * p + 1][s]);
        }
        // H_Q^T and S2^T = X2 X2_Q^T slice-partials
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                bf16x8 wb[TS];
                b8_from_acc<TS>(W2[2 * p][o], W2[2 * p + 1][o], wb);
                acc = mma32_terms<TS, TS>(acc, wb, x2qb[p]);
            }
            sm.hqp[w][o][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
        {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 2; ++p) acc = mma32_terms<TS, TS>(acc, x2b[p], x2qb[p]);
            sm.s2p[w][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
        // W1 += K^T (-Gt1) for this wave's columns
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            bf16x4 kt[TIN];
            load_kT_tile<S, TIN>(st.k, r, g, n, kt);
#pragma unroll
            for (int t = 0; t < 4; ++t) W1[r][t] = mma16_terms<TIN, TS>(W1[r][t], kt, g1n[t]);
        }
        __syncthreads();

        // ================= phase 3: H_Q, Z, the W2 updates =================
        bf16x4 g2n[4][TS];   // -Gt2[token 4g + j][output feature 16o + n]
#pragma unroll
        for (int o = 0; o < 4; ++o)
#pragma unroll
            for (int s = 0; s < TS; ++s) g2n[o][s] = tr4(sm.g2t[s], 4 * g + (n >> 2), 16 * o + 4 * (n & 3));
        bf16x4 s2b[TS];
        {
            float4 s = sm.s2p[0][lane];
#pragma unroll
            for (int ww = 1; ww < 4; ++ww) {
                const float4 u = sm.s2p[ww][lane];
                s = make_float4(s.x + u.x, s.y + u.y, s.z + u.z, s.w + u.w);
            }
            const float sv[4] = {s.x, s.y, s.z, s.w};
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (4 * g + i <= n) ? sv[i] : 0.f;
            terms4<TS>(x, s2b);
        }
        {
            // wave w forms H_Q^T tile w (output features 16w .. 16w + 15) and its
            // part of the output LayerNorm sums; the four parts meet in LDS
            const int o = w;
            float4 sq = sm.hqp[0][o][lane];
#pragma unroll
            for (int ww = 1; ww < 4; ++ww) {
                const float4 u = sm.hqp[ww][o][lane];
                sq = make_float4(sq.x + u.x, sq.y + u.y, sq.z + u.z, sq.w + u.w);
            }
            f32x4 hq = f32x4{sq.x, sq.y, sq.z, sq.w};
#pragma unroll
            for (int oo = 0; oo < 4; ++oo)                 // static indices into g2n
                if (oo == o) hq = mma16_terms<TS, TS>(hq, g2n[oo], s2b);   // - Gt2^T tril(S2)^T
            float p1 = (hq[0] + hq[1]) + (hq[2] + hq[3]);
            float p2 = fmaf(hq[0], hq[0], hq[1] * hq[1]) + fmaf(hq[2], hq[2], hq[3] * hq[3]);
            xrow4_sum2(p1, p2);
            if (g == 0) sm.xs[n][w] = make_float2(p1, p2);
            __syncthreads();
            const float2 x0 = sm.xs[n][0], x1 = sm.xs[n][1], x2 = sm.xs[n][2], x3 = sm.xs[n][3];
            const float s1 = (x0.x + x1.x) + (x2.x + x3.x), s2 = (x0.y + x1.y) + (x2.y + x3.y);
            const float mu = s1 * (1.f / D);
            const float rs = __builtin_amdgcn_rsqf(fmaxf(s2 * (1.f / D) - mu * mu, 0.f) + eps);
            if (n < bc) {
                const float4 qq = load4_f32<S>(st.q + n * STRIDE + 16 * o + 4 * g);
                const float4 ga = sm.gb[0][o][g], be = sm.gb[1][o][g];
                const float qv[4] = {qq.x, qq.y, qq.z, qq.w};
                const float gam[4] = {ga.x, ga.y, ga.z, ga.w}, bet[4] = {be.x, be.y, be.z, be.w};
                float z[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) z[i] = qv[i] + gam[i] * ((hq[i] - mu) * rs) + bet[i];
                *reinterpret_cast<float4*>(Zu + (size_t)(c * b + n) * D + 16 * o + 4 * g) =
                    make_float4(z[0], z[1], z[2], z[3]);
            }
        }
        // W2 += X2^T (-Gt2),  W2^T += (-Gt2)^T X2  (X2[token 4g + j][hidden hs + 16a + n])
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            bf16x4 x2n[TS];
#pragma unroll
            for (int s = 0; s < TS; ++s) x2n[s] = tr4(sm.x2t[w][s], 4 * g + (n >> 2), 16 * a + 4 * (n & 3));
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                W2[a][o] = mma16_terms<TS, TS>(W2[a][o], x2n, g2n[o]);
                W2T[o][a] = mma16_terms<TS, TS>(W2T[o][a], g2n[o], x2n);
            }
        }
        wave_lds_sync();   // this wave's tiles are rewritten by the next chunk
    }

    // ---- final state ----
    float* W1o = W1e + unit * (size_t)D * HID;
    float* W2o = W2e + unit * (size_t)HID * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) W1o[(16 * r + 4 * g + i) * HID + hs + 16 * t + n] = W1[r][t][i];
    // W2_end = W2_0 + (accumulated change): W2_0 - mean is formed with the rounding
    // it had at the start (W2_end may be W2_0: each entry is read and written by one lane)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float m = sm.w2m[w][16 * a + 4 * g + i];
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                const size_t idx = (size_t)(hs + 16 * a + 4 * g + i) * D + 16 * o + n;
                const float w0 = W2u[idx];
                W2o[idx] = w0 + (W2[a][o][i] - (w0 - m));
            }
        }
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
