// smallb_linear.hip -- TTT-Linear forward (plain and LayerNorm+residual inner
// model) for small mini-batches, d = 64, 1 <= b <= 16, fp32 token streams.
// (bf16 and two-term streams run the chain-on-one-wave kernel of
// smallb_chain.hip.)
//
// Method: web page "Test-Time Training: Linear Complexity Beyond Attention",
// sections "2. The Online Gradient Descent Update Rule", "3. Forward Evaluation
// and Output Projection" and "4. Mini-Batch Parallelism (Dual Formulation)".
// Per chunk c (rows Q, K, V, eta; state W_c):
//     H_K = K W_c,  G = d loss/d H_K (plain: 2(H_K - V); LN: LayerNorm backward
//     of 2(K + LN(H_K) - V)),  Gt = diag(eta) G
//     H_Q = Q W_c - tril(Q K^T) Gt,  Z = H_Q (plain) or Q + LN(H_Q)
//     W_{c+1} = W_c - K^T Gt
//
// Design (gfx950):
//  * One workgroup (4 waves) per (sequence, head) unit. Wave w owns the state
//    columns [16w, 16w+16) as four 16x16 fp32 MFMA accumulator tiles; W stays in
//    registers from the load of W0 to the store of W_end (the pages' "weight
//    update in SRAM" idea, page "How to Master Test-Time Training for Infinite
//    Context LLMs").
//  * The accumulator layout of W serves directly as the B operand of K W and
//    Q W (k index in the permuted order tile 2p rows 4g..4g+3, then tile 2p+1).
//    Passing the same registers as the A operand instead yields the transposed
//    product (W^T K^T): its C layout puts ONE token per lane (lane (g, n):
//    token n, features 16w+4g..16w+4g+3). The LayerNorm row statistics, the
//    per-token constants and the Z stores (16-byte vectors) are all done in
//    this "token per lane" layout: a row sum is three in-lane adds, two
//    permlane swaps and one 4-wave exchange through LDS.
//  * Gt is moved back to the MFMA C layout (token 4g+i, feature n) through a
//    per-wave LDS transpose; there it is the B operand of the state update
//    K^T Gt and (as Gt^T) the A operand of the causal term Gt^T tril(S)^T.
//  * S^T = K Q^T is computed so that its C layout is exactly the B operand of
//    Gt^T S^T.
//  * fp32 operands (state, gradient, scores) are split into bf16 terms: 3 next
//    to fp32 streams, which use 3 terms too (2 next to bf16 streams, for which
//    the template is still written).
//  * Q/K/V/eta chunks are prefetched PF chunks ahead into a register ring and
//    staged through double-buffered, row-padded LDS tiles. Per chunk: one
//    workgroup barrier (plain) or two (LayerNorm: forward statistics together
//    with the previous chunk's output statistics, then backward statistics).
#include "kernels.h"
#include "smallb_common.h"

namespace ttt {
namespace {

using namespace smallb;

template <typename S>
struct alignas(16) Smem {
    Stage<S> st[2];
    float red1[ROWS][4][4];         // [token][wave]: sum h, sum h^2 (chunk c), sum hq, sum hq^2 (chunk c-1)
    float red2[ROWS][4][2];         // [token][wave]: LayerNorm-backward sums
    float tp[4][ROWS][ROWS + 4];    // per-wave transpose tile [wave][feature][token]
    float wrow[4][D];               // LN kind: partial row sums of W0 over each wave's 16 columns
};

// Output stage of the LayerNorm kind for one chunk: Z = Q + LN(H_Q).
__device__ __forceinline__ void store_ln_out(float* __restrict__ Zu, const f32x4& hq, const float4& q,
                                             float s1, float s2, const float (&gam)[4],
                                             const float (&bet)[4], float eps, int c0, int bc, int n,
                                             int fcol)
{
    const float mu = s1 * (1.f / D);
    const float var = fmaxf(s2 * (1.f / D) - mu * mu, 0.f);
    const float rs = __builtin_amdgcn_rsqf(var + eps);
    const float qv[4] = {q.x, q.y, q.z, q.w};
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = qv[i] + gam[i] * ((hq[i] - mu) * rs) + bet[i];
    if (n < bc)
        *reinterpret_cast<float4*>(Zu + (size_t)(c0 + n) * D + fcol) = make_float4(z[0], z[1], z[2], z[3]);
}

template <int KIND, typename S, int TIN = Stor<S>::TERMS>
__global__ void __launch_bounds__(THREADS)
smallb_linear_kernel(int H, int N, int b, const S* __restrict__ Qg, const S* __restrict__ Kg,
                     const S* __restrict__ Vg, const float* __restrict__ etag, float eta_const,
                     const float* __restrict__ W0, const float* __restrict__ gamma,
                     const float* __restrict__ beta, float eps, float* __restrict__ Zg,
                     float* __restrict__ Wend)
{
    // TIN: terms of a token-stream operand; TS: terms of an fp32 operand (state,
    // gradient, scores): two next to exact bf16 or two-term streams, else three
    constexpr int TS = (TIN <= 2) ? 2 : 3;
    constexpr int STRIDE = Stor<S>::STRIDE;
    constexpr int PPT = (Pieces<S>::TOTAL + THREADS - 1) / THREADS;

    __shared__ Smem<S> sm;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int n = lane & 15;
    const int col = 16 * w + n;          // feature column in the MFMA C layout
    const int fcol = 16 * w + 4 * g;     // first of the four features in the token-per-lane layout

    const size_t unit = blockIdx.x;
    const int h = (int)(unit % H);
    const S* Qu = Qg + unit * (size_t)N * D;
    const S* Ku = Kg + unit * (size_t)N * D;
    const S* Vu = Vg + unit * (size_t)N * D;
    const float* etau = etag ? etag + unit * (size_t)N : nullptr;
    float* Zu = Zg + unit * (size_t)N * D;

    // ---- resident state: W[16r + 4g + i][col] ----
    f32x4 Wacc[4];
    {
        const float* W0u = W0 + unit * (size_t)D * D;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) Wacc[r][i] = W0u[(16 * r + 4 * g + i) * D + col];
    }
    float gam[4] = {0.f, 0.f, 0.f, 0.f}, bet[4] = {0.f, 0.f, 0.f, 0.f}, gam2x2[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KIND == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            gam[i] = gamma[h * D + fcol + i];
            bet[i] = beta[h * D + fcol + i];
            gam2x2[i] = 2.f * gam[i] * gam[i];
        }
    }

    const int nchunks = (N + b - 1) / b;

    // register ring: slot (c % PF) holds chunk c from its load until it is
    // written to LDS buffer (c & 1) during the processing of chunk c - 1
    uint4 pf[PF][PPT];
    float pe[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) pe[j] = 0.f;
    load_chunk<S, PPT>(pf[0], pe[0], 0, b, N, tid, Qu, Ku, Vu, etau, eta_const);
    store_chunk<S, PPT>(sm.st[0], pf[0], pe[0], tid, min(b, N));
#pragma unroll
    for (int j = 1; j <= PF; ++j)
        if (j < nchunks)
            load_chunk<S, PPT>(pf[j % PF], pe[j % PF], j, b, N, tid, Qu, Ku, Vu, etau, eta_const);

    // LN kind: the state is carried with each row's mean over the output
    // features removed (LayerNorm ignores a constant added to a whole row, and
    // its gradient sums to zero over the features, so the update never changes
    // the row means); the means are added back to W_end. Pre-activation rows
    // then have a near-zero mean whatever W0 holds, so the one-pass variance
    // keeps its relative precision.
    float wmean[4][4] = {};
    if constexpr (KIND == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s = row16_sum(Wacc[r][i]);
                if (n == 0) sm.wrow[w][16 * r + 4 * g + i] = s;
            }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * r + 4 * g + i;
                wmean[r][i] = ((sm.wrow[0][row] + sm.wrow[1][row]) + (sm.wrow[2][row] + sm.wrow[3][row])) * (1.f / D);
                Wacc[r][i] -= wmean[r][i];
            }
    }

    // W_c as B-operand terms, permuted k order
    bf16x8 Wb[2][TS];
#pragma unroll
    for (int p = 0; p < 2; ++p) b8_from_acc<TS>(Wacc[2 * p], Wacc[2 * p + 1], Wb[p]);

    // previous chunk's output, waiting for its LayerNorm statistics
    f32x4 hq_prev = {0.f, 0.f, 0.f, 0.f};
    float4 q_prev = make_float4(0.f, 0.f, 0.f, 0.f);
    int c0_prev = 0, bc_prev = 0;

    __syncthreads();

    for (int cb = 0; cb < nchunks; cb += PF) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const int c = cb + j;
            if (c < nchunks) {
                const int c0 = c * b;
                const int bc = min(b, N - c0);
                const Stage<S>& st = sm.st[c & 1];
                const int nslot = (j + 1) % PF;   // ring slot of chunk c + 1

                // ======== phase A: operands and products of chunk c ========
                bf16x8 ka[2][TIN], qa[2][TIN];
                f32x4 sT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int o0 = n * STRIDE + 32 * p + 4 * g;
                    load_a8<S, TIN>(st.k + o0, st.k + o0 + 16, ka[p]);
                    load_a8<S, TIN>(st.q + o0, st.q + o0 + 16, qa[p]);
                    bf16x8 kn[TIN], qn[TIN];
                    const int o1 = n * STRIDE + 32 * p + 8 * g;
                    load_a8<S, TIN>(st.k + o1, st.k + o1 + 4, kn);
                    load_a8<S, TIN>(st.q + o1, st.q + o1 + 4, qn);
                    sT = mma32_terms<TIN, TIN>(sT, kn, qn);   // lane (g,n): S[n][4g+i]
                }
                bf16x4 kt[4][TIN];
#pragma unroll
                for (int r = 0; r < 4; ++r) load_kT_tile<S, TIN>(st.k, r, g, n, kt[r]);
                const float4 qT = load4_f32<S>(st.q + n * STRIDE + fcol);

                // H_Q^T (token per lane)
                f32x4 hqT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 2; ++p) hqT = mma32_terms<TS, TIN>(hqT, Wb[p], qa[p]);

                float gt[4];   // diag(eta) G in the MFMA C layout (token 4g+i, feature col)
                if constexpr (KIND == 0) {
                    f32x4 hk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int p = 0; p < 2; ++p) hk = mma32_terms<TIN, TS>(hk, ka[p], Wb[p]);
                    const float4 et = *reinterpret_cast<const float4*>(st.eta + 4 * g);
                    const float etv[4] = {et.x, et.y, et.z, et.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float vv = Stor<S>::f(st.v[(4 * g + i) * STRIDE + col]);
                        gt[i] = (4 * g + i < bc) ? 2.f * etv[i] * (hk[i] - vv) : 0.f;
                    }
                    // chunk c+1 into LDS, refill its ring slot
                    if (c + 1 < nchunks) {
                        store_chunk<S, PPT>(sm.st[(c + 1) & 1], pf[nslot], pe[nslot], tid,
                                            min(b, N - (c + 1) * b));
                        if (c + 1 + PF < nchunks)
                            load_chunk<S, PPT>(pf[nslot], pe[nslot], c + 1 + PF, b, N, tid, Qu, Ku,
                                               Vu, etau, eta_const);
                    }
                } else {
                    // H_K^T (token per lane) and LayerNorm forward partial sums
                    f32x4 hkT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int p = 0; p < 2; ++p) hkT = mma32_terms<TS, TIN>(hkT, Wb[p], ka[p]);
                    const float4 kT = load4_f32<S>(st.k + n * STRIDE + fcol);
                    const float4 vT = load4_f32<S>(st.v + n * STRIDE + fcol);
                    const float eta_n = st.eta[n];
                    const float kv[4] = {kT.x - vT.x, kT.y - vT.y, kT.z - vT.z, kT.w - vT.w};
                    float cpr[4];   // 2 gamma (K - V + beta): residual part of 2 E gamma
#pragma unroll
                    for (int i = 0; i < 4; ++i) cpr[i] = 2.f * gam[i] * (kv[i] + bet[i]);

                    float s1 = (hkT[0] + hkT[1]) + (hkT[2] + hkT[3]);
                    float s2 = (hkT[0] * hkT[0] + hkT[1] * hkT[1]) + (hkT[2] * hkT[2] + hkT[3] * hkT[3]);
                    float s3 = (hq_prev[0] + hq_prev[1]) + (hq_prev[2] + hq_prev[3]);
                    float s4 = (hq_prev[0] * hq_prev[0] + hq_prev[1] * hq_prev[1]) +
                               (hq_prev[2] * hq_prev[2] + hq_prev[3] * hq_prev[3]);
                    s1 = xrow4_sum(s1);
                    s2 = xrow4_sum(s2);
                    s3 = xrow4_sum(s3);
                    s4 = xrow4_sum(s4);
                    if (g == 0)
                        *reinterpret_cast<float4*>(&sm.red1[n][w][0]) = make_float4(s1, s2, s3, s4);
                    // chunk c+1 into LDS, refill its ring slot
                    if (c + 1 < nchunks) {
                        store_chunk<S, PPT>(sm.st[(c + 1) & 1], pf[nslot], pe[nslot], tid,
                                            min(b, N - (c + 1) * b));
                        if (c + 1 + PF < nchunks)
                            load_chunk<S, PPT>(pf[nslot], pe[nslot], c + 1 + PF, b, N, tid, Qu, Ku,
                                               Vu, etau, eta_const);
                    }
                    __syncthreads();   // X1

                    // ======== phase B: forward statistics, backward partial sums ========
                    float t[4][4];
#pragma unroll
                    for (int ww = 0; ww < 4; ++ww) {
                        const float4 v = *reinterpret_cast<const float4*>(&sm.red1[n][ww][0]);
                        t[ww][0] = v.x;
                        t[ww][1] = v.y;
                        t[ww][2] = v.z;
                        t[ww][3] = v.w;
                    }
                    const float S1 = (t[0][0] + t[1][0]) + (t[2][0] + t[3][0]);
                    const float S2 = (t[0][1] + t[1][1]) + (t[2][1] + t[3][1]);
                    const float S3 = (t[0][2] + t[1][2]) + (t[2][2] + t[3][2]);
                    const float S4 = (t[0][3] + t[1][3]) + (t[2][3] + t[3][3]);
                    const float mu = S1 * (1.f / D);
                    const float rs = __builtin_amdgcn_rsqf(fmaxf(S2 * (1.f / D) - mu * mu, 0.f) + eps);
                    float xh[4], dxh[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xh[i] = (hkT[i] - mu) * rs;
                        dxh[i] = cpr[i] + gam2x2[i] * xh[i];
                    }
                    float u1 = (dxh[0] + dxh[1]) + (dxh[2] + dxh[3]);
                    float u2 = (dxh[0] * xh[0] + dxh[1] * xh[1]) + (dxh[2] * xh[2] + dxh[3] * xh[3]);
                    u1 = xrow4_sum(u1);
                    u2 = xrow4_sum(u2);
                    if (g == 0) *reinterpret_cast<float2*>(&sm.red2[n][w][0]) = make_float2(u1, u2);
                    if (c > 0)
                        store_ln_out(Zu, hq_prev, q_prev, S3, S4, gam, bet, eps, c0_prev, bc_prev, n,
                                     fcol);
                    __syncthreads();   // X2

                    // ======== phase C: gradient, moved to the MFMA C layout ========
                    const float4 a = *reinterpret_cast<const float4*>(&sm.red2[n][0][0]);
                    const float4 bb = *reinterpret_cast<const float4*>(&sm.red2[n][2][0]);
                    const float m1 = ((a.x + a.z) + (bb.x + bb.z)) * (1.f / D);
                    const float m2 = ((a.y + a.w) + (bb.y + bb.w)) * (1.f / D);
                    const float scale = eta_n * rs;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sm.tp[w][4 * g + i][n] = (n < bc) ? scale * (dxh[i] - m1 - xh[i] * m2) : 0.f;
                    // the tile is private to this wave: order its LDS writes before the reads
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    const float4 gv = *reinterpret_cast<const float4*>(&sm.tp[w][n][4 * g]);
                    gt[0] = gv.x;
                    gt[1] = gv.y;
                    gt[2] = gv.z;
                    gt[3] = gv.w;
                }

                // -Gt as terms: B operand of K^T Gt (k = token), A operand of Gt^T S^T
                bf16x4 ngb[TS];
                {
                    float x[4] = {-gt[0], -gt[1], -gt[2], -gt[3]};
                    terms4<TS>(x, ngb);
                }
                // H_Q^T -= Gt^T tril(S)^T
                {
                    float x[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = (4 * g + i <= n) ? sT[i] : 0.f;
                    bf16x4 sb[TS];
                    terms4<TS>(x, sb);
                    hqT = mma16_terms<TS, TS>(hqT, ngb, sb);
                }
                // W_{c+1} = W_c - K^T Gt
#pragma unroll
                for (int r = 0; r < 4; ++r) Wacc[r] = mma16_terms<TIN, TS>(Wacc[r], kt[r], ngb);
#pragma unroll
                for (int p = 0; p < 2; ++p) b8_from_acc<TS>(Wacc[2 * p], Wacc[2 * p + 1], Wb[p]);

                if constexpr (KIND == 0) {
                    if (n < bc)
                        *reinterpret_cast<float4*>(Zu + (size_t)(c0 + n) * D + fcol) =
                            make_float4(hqT[0], hqT[1], hqT[2], hqT[3]);
                    __syncthreads();   // chunk c+1 staged
                } else {
                    hq_prev = hqT;
                    q_prev = qT;
                    c0_prev = c0;
                    bc_prev = bc;
                }
            }
        }
    }

    if constexpr (KIND == 1) {
        // output statistics of the last chunk
        float s3 = (hq_prev[0] + hq_prev[1]) + (hq_prev[2] + hq_prev[3]);
        float s4 = (hq_prev[0] * hq_prev[0] + hq_prev[1] * hq_prev[1]) +
                   (hq_prev[2] * hq_prev[2] + hq_prev[3] * hq_prev[3]);
        s3 = xrow4_sum(s3);
        s4 = xrow4_sum(s4);
        // red1 is free: every wave has passed the last chunk's X2 barrier
        if (g == 0) *reinterpret_cast<float2*>(&sm.red1[n][w][0]) = make_float2(s3, s4);
        __syncthreads();
        float S3 = 0.f, S4 = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float2 v = *reinterpret_cast<const float2*>(&sm.red1[n][ww][0]);
            S3 += v.x;
            S4 += v.y;
        }
        store_ln_out(Zu, hq_prev, q_prev, S3, S4, gam, bet, eps, c0_prev, bc_prev, n, fcol);
    }

    // W_end = W0 + (accumulated change): W0 - mean is formed again with the
    // rounding it had at the start, so a state that never moved comes back bit
    // for bit. (W_end may be W0: every entry is read and written by one lane.)
    float* Wu = Wend + unit * (size_t)D * D;
    const float* W0u = W0 + unit * (size_t)D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const size_t o = (size_t)(16 * r + 4 * g + i) * D + col;
            float v = Wacc[r][i];
            if constexpr (KIND == 1) {
                const float w0 = W0u[o];
                v = w0 + (v - (w0 - wmean[r][i]));
            }
            Wu[o] = v;
        }
}

template <int KIND, typename S, int TIN = Stor<S>::TERMS>
hipError_t launch_typed(const LinearArgs& a, hipStream_t stream)
{
    const int units = a.B * a.H;
    hipLaunchKernelGGL((smallb_linear_kernel<KIND, S, TIN>), dim3(units), dim3(THREADS), 0, stream, a.H,
                       a.N, a.b, static_cast<const S*>(a.Q), static_cast<const S*>(a.K),
                       static_cast<const S*>(a.V), a.eta, a.eta_const, a.W0, a.gamma, a.beta,
                       a.eps, a.Z, a.W_end);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_smallb_linear(const LinearArgs& a, hipStream_t stream)
{
    if (a.d != D || a.b > ROWS) return launch_midb_linear(a, stream);
    if (a.dtype == 1) return launch_smallb_chain(a, stream);
    return a.kind == 1 ? launch_typed<1, float>(a, stream) : launch_typed<0, float>(a, stream);
}

}  // namespace ttt
