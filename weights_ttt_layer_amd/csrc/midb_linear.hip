// midb_linear.hip -- TTT-Linear forward (plain and LayerNorm+residual inner
// model) for the combinations the two specialised small-b kernels do not
// take: chunks of 17..64 tokens at head dimension 64, and head dimension 128
// with chunks of 1..64 tokens; fp32 or bf16 token streams.
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
// Design (gfx950): one workgroup of four waves per (sequence, head) unit.
//  * Wave w keeps the state columns 64t + 16w .. 64t + 16w + 15 (t < D/64) for
//    the whole scan as D/16 x D/64 fp32 MFMA accumulator tiles (rows = input
//    features): W never leaves the chip between W0 and W_end.
//  * A chunk of up to 16 NG rows is handled as NG groups of 16 tokens. The
//    accumulator tiles, split into bf16 terms, are the A operand of W^T K^T and
//    W^T Q^T (one token per lane: the LayerNorm row statistics are in-lane adds,
//    two lane swaps and a four-wave exchange through LDS) and the B operand of
//    K W (plain: the gradient directly in the MFMA C layout).
//  * The LayerNorm gradient goes back to the C layout through a per-wave LDS
//    transpose; there it is the B operand of the update K^T Gt and the A operand
//    of the causal term Gt^T tril(S)^T, S^T = K Q^T per pair of groups.
//  * Precision as in the other small-b kernels: fp32 operands (state, gradient,
//    scores) as two bf16 terms next to bf16 streams, three next to fp32 streams
//    (which use three terms too); fp32 accumulation.
//  * LN kind: the state is carried with each row's mean over the output
//    features removed (LayerNorm ignores a constant added to a whole row and
//    its gradient sums to zero over the features, so the update never moves
//    the row means); W_end = W0 + (accumulated change).
//  * One LDS stage holds the chunk's Q, K, V, eta; the next chunk waits in
//    registers (issued one chunk ahead) where they fit.
#include "kernels.h"
#include "smallb_common.h"

namespace ttt {
namespace {

using smallb::b8_from_acc;
using smallb::load4_f32;
using smallb::load_a8;

constexpr int MB_THREADS = 256;

template <typename S> struct MStor;
template <> struct MStor<uint16_t> {
    static constexpr int TERMS = 1;
    static constexpr int PAD = 8;      // elements: rows of 144 / 272 bytes
};
template <> struct MStor<float> {
    static constexpr int TERMS = 3;
    static constexpr int PAD = 4;      // rows of 272 / 528 bytes
};

template <int D, int NG, typename S>
struct MidGeom {
    static constexpr int ROWS = 16 * NG;
    static constexpr int STRIDE = D + MStor<S>::PAD;
    static constexpr int PIECES = D * (int)sizeof(S) / 16;   // 16-byte pieces per row
    static constexpr int TOTAL = 3 * ROWS * PIECES;
    static constexpr int PPT = (TOTAL + MB_THREADS - 1) / MB_THREADS;
    // the next chunk waits in registers when it takes at most 12 pieces a thread
    static constexpr bool PREFETCH = PPT <= 12;
};

template <int D, int NG, typename S>
struct alignas(16) MidSmem {
    using G = MidGeom<D, NG, S>;
    S q[G::ROWS * G::STRIDE];
    S k[G::ROWS * G::STRIDE];
    S v[G::ROWS * G::STRIDE];
    float eta[G::ROWS];
    float rf[G::ROWS][4][2];    // LayerNorm forward partial sums [token][wave]
    float rb[G::ROWS][4][2];    // LayerNorm backward partial sums
    float ro[G::ROWS][4][2];    // output LayerNorm partial sums
    float tp[4][16][20];        // per-wave transpose tile [wave][feature][token]
    float wrow[4][D];           // LN kind: partial row sums of W0
};

// Global loads of chunk c (rows clamped into the sequence; rows past its end
// are zeroed when the tile is written to LDS).
template <int D, int NG, typename S, int PPT>
__device__ __forceinline__ void mid_load(uint4 (&pf)[PPT], float& pe, int c0, int N, int tid, const S* Qu,
                                         const S* Ku, const S* Vu, const float* etau, float eta_const)
{
    using G = MidGeom<D, NG, S>;
    static_assert(PPT == G::PPT, "pieces per thread");
#pragma unroll
    for (int k = 0; k < G::PPT; ++k) {
        const int idx = min(tid + k * MB_THREADS, G::TOTAL - 1);
        const int tensor = idx / (G::ROWS * G::PIECES);
        const int rem = idx - tensor * (G::ROWS * G::PIECES);
        const int row = rem / G::PIECES;
        const int piece = rem - row * G::PIECES;
        const S* src = tensor == 0 ? Qu : (tensor == 1 ? Ku : Vu);
        const int srow = min(c0 + row, N - 1);
        pf[k] = *reinterpret_cast<const uint4*>(src + (size_t)srow * D + piece * (16 / (int)sizeof(S)));
    }
    pe = etau ? etau[min(c0 + tid % G::ROWS, N - 1)] : eta_const;
}

template <int D, int NG, typename S, int PPT>
__device__ __forceinline__ void mid_store(MidSmem<D, NG, S>& sm, const uint4 (&pf)[PPT], float pe, int tid, int bc)
{
    using G = MidGeom<D, NG, S>;
    static_assert(PPT == G::PPT, "pieces per thread");
#pragma unroll
    for (int k = 0; k < G::PPT; ++k) {
        const int idx = tid + k * MB_THREADS;
        if (idx < G::TOTAL) {
            const int tensor = idx / (G::ROWS * G::PIECES);
            const int rem = idx - tensor * (G::ROWS * G::PIECES);
            const int row = rem / G::PIECES;
            const int piece = rem - row * G::PIECES;
            S* dst = tensor == 0 ? sm.q : (tensor == 1 ? sm.k : sm.v);
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
            *reinterpret_cast<uint4*>(dst + row * G::STRIDE + piece * (16 / (int)sizeof(S))) = row < bc ? pf[k] : z;
        }
    }
    if (tid < G::ROWS) sm.eta[tid] = tid < bc ? pe : 0.f;
}

// A operand (16x16x16) of K^T for feature tile r of the 16 rows at `k`: lane
// (g, n) gets K[4g + j][16r + n], j = 0..3.
template <typename S, int T, int STRIDE>
__device__ __forceinline__ void kT_tile(const S* k, int r, int g, int n, bf16x4 (&out)[T])
{
    if constexpr (sizeof(S) == 2) {
        static_assert(T == 1, "bf16 streams are exact in one term");
        typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
        const S* p = k + (4 * g + (n >> 2)) * STRIDE + 16 * r + 4 * (n & 3);
        out[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(p));
    } else {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = k[(4 * g + j) * STRIDE + 16 * r + n];
        terms4<T>(x, out);
    }
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// BIG: chunks longer than one block of 16 NG rows (plain f only). A chunk is
// then a sequence of blocks: every block's gradient is taken at the chunk-start
// state W_c (kept as a second copy), its outputs use the running state W' that
// already holds the updates of the chunk's earlier blocks, and W' takes the
// block's update; W' is W_{c+1} once the chunk ends. (The dual form's causal
// sum over the chunk, split at block boundaries by associativity.)
// APPLY (BIG only): the block-causal outputs of page "Test-Time Training Done
// Right" (abstract) instead of the dual form's: every output of chunk c is
// f(Q; W_c) (APPLY_BEFORE: the products with Q take W_c, no causal term) or
// f(Q; W_{c+1}) (APPLY_AFTER: once the chunk's last block has stepped the
// state, its Q rows are read again, block by block, against W_{c+1}).
enum { APPLY_DUAL = 0, APPLY_BEFORE = 1, APPLY_AFTER = 2 };

template <int D, int NG, int KIND, typename S, bool BIG, int APPLY>
__global__ void __launch_bounds__(MB_THREADS)
midb_linear_kernel(int H, int N, int b, const S* __restrict__ Qg, const S* __restrict__ Kg,
                   const S* __restrict__ Vg, const float* __restrict__ etag, float eta_const,
                   const float* __restrict__ W0, const float* __restrict__ gamma, const float* __restrict__ beta,
                   float eps, float* __restrict__ Zg, float* __restrict__ Wend)
{
    using G = MidGeom<D, NG, S>;
    static_assert(!BIG || KIND == 0, "blocks of a longer chunk: plain f only");
    static_assert(APPLY == APPLY_DUAL || BIG, "block-causal outputs: blocks of a longer chunk");
    constexpr int CT = D / 64;          // column tiles per wave
    constexpr int RT = D / 16;          // row tiles of the state
    constexpr int KS = D / 32;          // 16x16x32 steps over the features
    constexpr int TIN = MStor<S>::TERMS;
    constexpr int TS = (TIN == 1) ? 2 : 3;
    constexpr int ST = G::STRIDE;

    __shared__ MidSmem<D, NG, S> sm;

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
    const float* W0u = W0 + unit * (size_t)D * D;

    // ---- resident state: Wacc[r][t][i] = W[16r + 4g + i][64t + 16w + n] ----
    f32x4 Wacc[RT][CT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) Wacc[r][t][i] = W0u[(16 * r + 4 * g + i) * D + 64 * t + 16 * w + n];

    // LayerNorm parameters of this lane's features 64t + 16w + 4g + i (token-per-lane layout)
    float gam[CT][4] = {}, bet[CT][4] = {};
    if constexpr (KIND == 1) {
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gam[t][i] = gamma[h * D + 64 * t + 16 * w + 4 * g + i];
                bet[t][i] = beta[h * D + 64 * t + 16 * w + 4 * g + i];
            }
    }

    // LN kind: remove each state row's mean over the output features (the means
    // stay in LDS and are formed again, identically, for W_end)
    auto row_mean = [&](int row) {
        return ((sm.wrow[0][row] + sm.wrow[1][row]) + (sm.wrow[2][row] + sm.wrow[3][row])) * (1.f / D);
    };
    if constexpr (KIND == 1) {
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float s = 0.f;
#pragma unroll
                for (int t = 0; t < CT; ++t) s += Wacc[r][t][i];
                s = row16_sum(s);
                if (n == 0) sm.wrow[w][16 * r + 4 * g + i] = s;
            }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float m = row_mean(16 * r + 4 * g + i);
#pragma unroll
                for (int t = 0; t < CT; ++t) Wacc[r][t][i] -= m;
            }
    }

    // Blocks of at most ROWS tokens, in order: chunk c covers rows [c b, c b + b);
    // a block never crosses a chunk boundary (without BIG, a block is a chunk).
    auto block_rows = [&](int r0) {            // rows of the block starting at row r0
        const int cend = min((r0 / b + 1) * b, N);
        return min(G::ROWS, cend - r0);
    };
    f32x4 Wc[BIG ? RT : 1][BIG ? CT : 1];      // BIG: W_c, the chunk-start state
    uint4 pf[G::PPT];
    float pe = 0.f;
    mid_load<D, NG, S, G::PPT>(pf, pe, 0, N, tid, Qu, Ku, Vu, etau, eta_const);
    mid_store<D, NG, S, G::PPT>(sm, pf, pe, tid, block_rows(0));
    if constexpr (G::PREFETCH)
        if (block_rows(0) < N) mid_load<D, NG, S, G::PPT>(pf, pe, block_rows(0), N, tid, Qu, Ku, Vu, etau, eta_const);
    __syncthreads();

    for (int c0 = 0; c0 < N;) {
        const int bc = block_rows(c0);
        const int c1 = c0 + bc;                // next block's first row
        if constexpr (BIG) {
            if (c0 % b == 0) {
#pragma unroll
                for (int r = 0; r < RT; ++r)
#pragma unroll
                    for (int t = 0; t < CT; ++t) Wc[r][t] = Wacc[r][t];
            }
        }

        // ======== products at W_c ========
        // W_c as operand terms: lane (g, n) holds W[32p + 4g + i (+16)][64t + 16w + n]
        f32x4 hqT[NG][CT];       // (Q W)^T: lane (g, n) = token n of the group, features 64t + 16w + 4g + i
        f32x4 hk[NG][CT];        // LN: (K W)^T as hqT; plain: K W in the C layout (token 4g + i, feature 64t + 16w + n)
#pragma unroll
        for (int t = 0; t < CT; ++t) {
            // column tile t of W_c as operand terms: lane (g, n) holds W[32p + 4g + i (+16)][64t + 16w + n]
            // (BIG: Wb is the running state W' for the outputs, Wg the chunk-start W_c for the gradient)
            bf16x8 Wb[APPLY == APPLY_DUAL ? KS : 1][TS];
            if constexpr (APPLY == APPLY_DUAL) {
#pragma unroll
                for (int p = 0; p < KS; ++p) b8_from_acc<TS>(Wacc[2 * p][t], Wacc[2 * p + 1][t], Wb[p]);
            }
            bf16x8 Wg[BIG ? KS : 1][TS];
            if constexpr (BIG) {
#pragma unroll
                for (int p = 0; p < KS; ++p) b8_from_acc<TS>(Wc[2 * p][t], Wc[2 * p + 1][t], Wg[p]);
            }
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                hqT[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
                hk[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < KS; ++p) {
                    const int o = (16 * j + n) * ST + 32 * p + 4 * g;
                    bf16x8 qa[TIN], ka[TIN];
                    load_a8<S, TIN>(sm.q + o, sm.q + o + 16, qa);
                    load_a8<S, TIN>(sm.k + o, sm.k + o + 16, ka);
                    if constexpr (APPLY == APPLY_DUAL)
                        hqT[j][t] = mma32_terms<TS, TIN>(hqT[j][t], Wb[p], qa);
                    else if constexpr (APPLY == APPLY_BEFORE)
                        hqT[j][t] = mma32_terms<TS, TIN>(hqT[j][t], Wg[p], qa);
                    if constexpr (KIND == 1)
                        hk[j][t] = mma32_terms<TS, TIN>(hk[j][t], Wb[p], ka);
                    else if constexpr (BIG)
                        hk[j][t] = mma32_terms<TIN, TS>(hk[j][t], ka, Wg[p]);
                    else
                        hk[j][t] = mma32_terms<TIN, TS>(hk[j][t], ka, Wb[APPLY == APPLY_DUAL ? p : 0]);
                }
            }
        }

        // ======== gradient, in the MFMA C layout: gt[j][t][i] = Gt[16j + 4g + i][64t + 16w + n] ========
        float gt[NG][CT][4];
        if constexpr (KIND == 0) {
#pragma unroll
            for (int j = 0; j < NG; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * j + 4 * g + i;
                    const float e = 2.f * sm.eta[row];
#pragma unroll
                    for (int t = 0; t < CT; ++t) {
                        const float vv = smallb::Stor<S>::f(sm.v[row * ST + 64 * t + 16 * w + n]);
                        gt[j][t][i] = e * (hk[j][t][i] - vv);
                    }
                }
        } else {
            // LayerNorm forward statistics
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                float s1 = 0.f, s2 = 0.f;
#pragma unroll
                for (int t = 0; t < CT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        s1 += hk[j][t][i];
                        s2 = fmaf(hk[j][t][i], hk[j][t][i], s2);
                    }
                xrow4_sum2(s1, s2);
                if (g == 0) *reinterpret_cast<float2*>(&sm.rf[16 * j + n][w][0]) = make_float2(s1, s2);
            }
            __syncthreads();
            // x-hat and gamma * d loss / d LN = 2 gamma (K + gamma x-hat + beta - V), formed
            // twice (for the backward sums, then for the gradient) rather than kept
            float mu[NG], rs[NG];
            auto xh_dx = [&](int j, int t, float (&xh)[4], float (&dx)[4]) {
                const int f = 64 * t + 16 * w + 4 * g;
                const float4 kk = load4_f32<S>(sm.k + (16 * j + n) * ST + f);
                const float4 vv = load4_f32<S>(sm.v + (16 * j + n) * ST + f);
                const float kv[4] = {kk.x - vv.x, kk.y - vv.y, kk.z - vv.z, kk.w - vv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xh[i] = (hk[j][t][i] - mu[j]) * rs[j];
                    dx[i] = 2.f * gam[t][i] * (kv[i] + gam[t][i] * xh[i] + bet[t][i]);
                }
            };
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                const float4 a = *reinterpret_cast<const float4*>(&sm.rf[16 * j + n][0][0]);
                const float4 bb = *reinterpret_cast<const float4*>(&sm.rf[16 * j + n][2][0]);
                mu[j] = ((a.x + a.z) + (bb.x + bb.z)) * (1.f / D);
                const float ms = ((a.y + a.w) + (bb.y + bb.w)) * (1.f / D);
                rs[j] = __builtin_amdgcn_rsqf(fmaxf(ms - mu[j] * mu[j], 0.f) + eps);
                float u1 = 0.f, u2 = 0.f;
#pragma unroll
                for (int t = 0; t < CT; ++t) {
                    float xh[4], dx[4];
                    xh_dx(j, t, xh, dx);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        u1 += dx[i];
                        u2 = fmaf(dx[i], xh[i], u2);
                    }
                }
                xrow4_sum2(u1, u2);
                if (g == 0) *reinterpret_cast<float2*>(&sm.rb[16 * j + n][w][0]) = make_float2(u1, u2);
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                const float4 a = *reinterpret_cast<const float4*>(&sm.rb[16 * j + n][0][0]);
                const float4 bb = *reinterpret_cast<const float4*>(&sm.rb[16 * j + n][2][0]);
                const float m1 = ((a.x + a.z) + (bb.x + bb.z)) * (1.f / D);
                const float m2 = ((a.y + a.w) + (bb.y + bb.w)) * (1.f / D);
                const float scale = sm.eta[16 * j + n] * rs[j];
#pragma unroll
                for (int t = 0; t < CT; ++t) {
                    float xh[4], dx[4];
                    xh_dx(j, t, xh, dx);
                    // token n, features 4g + i of the tile -> token 4g + i, feature n
#pragma unroll
                    for (int i = 0; i < 4; ++i) sm.tp[w][4 * g + i][n] = scale * (dx[i] - m1 - xh[i] * m2);
                    wave_lds_sync();
                    const float4 gv = *reinterpret_cast<const float4*>(&sm.tp[w][n][4 * g]);
                    gt[j][t][0] = gv.x;
                    gt[j][t][1] = gv.y;
                    gt[j][t][2] = gv.z;
                    gt[j][t][3] = gv.w;
                    wave_lds_sync();
                }
            }
        }

        // -Gt as terms: B operand of K^T Gt (k = token), A operand of Gt^T S^T
        bf16x4 ngb[NG][CT][TS];
#pragma unroll
        for (int j = 0; j < NG; ++j)
#pragma unroll
            for (int t = 0; t < CT; ++t) {
                float x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = (16 * j + 4 * g + i < bc) ? -gt[j][t][i] : 0.f;
                terms4<TS>(x, ngb[j][t]);
            }

        // ======== causal term: H_Q^T(group jq) -= sum_{jk <= jq} Gt_jk^T tril(S)^T ========
#pragma unroll
        for (int jq = 0; jq < (APPLY == APPLY_DUAL ? NG : 0); ++jq)
#pragma unroll
            for (int jk = 0; jk <= jq; ++jk) {
                // S^T block: lane (g, n) holds S[query 16jq + n][key 16jk + 4g + i] = q . k
                f32x4 sT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < KS; ++p) {
                    bf16x8 kn[TIN], qn[TIN];
                    const int ok = (16 * jk + n) * ST + 32 * p + 8 * g;
                    const int oq = (16 * jq + n) * ST + 32 * p + 8 * g;
                    load_a8<S, TIN>(sm.k + ok, sm.k + ok + 4, kn);
                    load_a8<S, TIN>(sm.q + oq, sm.q + oq + 4, qn);
                    sT = mma32_terms<TIN, TIN>(sT, kn, qn);
                }
                float x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = (jk < jq || 4 * g + i <= n) ? sT[i] : 0.f;
                bf16x4 sb[TS];
                terms4<TS>(x, sb);
#pragma unroll
                for (int t = 0; t < CT; ++t) hqT[jq][t] = mma16_terms<TS, TS>(hqT[jq][t], ngb[jk][t], sb);
            }

        // ======== W_{c+1} = W_c - K^T Gt ========
#pragma unroll
        for (int j = 0; j < NG; ++j)
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                bf16x4 kt[TIN];
                kT_tile<S, TIN, ST>(sm.k + 16 * j * ST, r, g, n, kt);
#pragma unroll
                for (int t = 0; t < CT; ++t) Wacc[r][t] = mma16_terms<TIN, TS>(Wacc[r][t], kt, ngb[j][t]);
            }

        // ======== outputs ========
        if constexpr (APPLY == APPLY_AFTER) {
            // the chunk's outputs once its last block has stepped the state
            if (c1 % b == 0 || c1 == N) {
                __syncthreads();                   // every wave is done with this block's stage
                const int cs = (c0 / b) * b;       // the chunk's first row
                for (int r0 = cs; r0 < c1; r0 += G::ROWS) {
                    const int rows = min(G::ROWS, c1 - r0);
                    for (int idx = tid; idx < G::ROWS * G::PIECES; idx += MB_THREADS) {
                        const int row = idx / G::PIECES, piece = idx - row * G::PIECES;
                        uint4 val = make_uint4(0u, 0u, 0u, 0u);
                        if (row < rows)
                            val = *reinterpret_cast<const uint4*>(Qu + (size_t)(r0 + row) * D +
                                                                  piece * (16 / (int)sizeof(S)));
                        *reinterpret_cast<uint4*>(sm.q + row * G::STRIDE + piece * (16 / (int)sizeof(S))) = val;
                    }
                    __syncthreads();
#pragma unroll
                    for (int t = 0; t < CT; ++t) {
                        bf16x8 Wn[KS][TS];         // W_{c+1}
#pragma unroll
                        for (int p = 0; p < KS; ++p) b8_from_acc<TS>(Wacc[2 * p][t], Wacc[2 * p + 1][t], Wn[p]);
#pragma unroll
                        for (int j = 0; j < NG; ++j) {
                            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int p = 0; p < KS; ++p) {
                                const int o = (16 * j + n) * ST + 32 * p + 4 * g;
                                bf16x8 qa[TIN];
                                load_a8<S, TIN>(sm.q + o, sm.q + o + 16, qa);
                                acc = mma32_terms<TS, TIN>(acc, Wn[p], qa);
                            }
                            if (16 * j + n < rows)
                                *reinterpret_cast<float4*>(Zu + (size_t)(r0 + 16 * j + n) * D + 64 * t + 16 * w +
                                                           4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
                        }
                    }
                    __syncthreads();               // the stage's Q rows are read again
                }
            }
        } else if constexpr (KIND == 0) {
#pragma unroll
            for (int j = 0; j < NG; ++j)
                if (16 * j + n < bc)
#pragma unroll
                    for (int t = 0; t < CT; ++t)
                        *reinterpret_cast<float4*>(Zu + (size_t)(c0 + 16 * j + n) * D + 64 * t + 16 * w + 4 * g) =
                            make_float4(hqT[j][t][0], hqT[j][t][1], hqT[j][t][2], hqT[j][t][3]);
        } else {
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                float s1 = 0.f, s2 = 0.f;
#pragma unroll
                for (int t = 0; t < CT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        s1 += hqT[j][t][i];
                        s2 = fmaf(hqT[j][t][i], hqT[j][t][i], s2);
                    }
                xrow4_sum2(s1, s2);
                if (g == 0) *reinterpret_cast<float2*>(&sm.ro[16 * j + n][w][0]) = make_float2(s1, s2);
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                const float4 a = *reinterpret_cast<const float4*>(&sm.ro[16 * j + n][0][0]);
                const float4 bb = *reinterpret_cast<const float4*>(&sm.ro[16 * j + n][2][0]);
                const float mu = ((a.x + a.z) + (bb.x + bb.z)) * (1.f / D);
                const float ms = ((a.y + a.w) + (bb.y + bb.w)) * (1.f / D);
                const float r = __builtin_amdgcn_rsqf(fmaxf(ms - mu * mu, 0.f) + eps);
                if (16 * j + n < bc) {
#pragma unroll
                    for (int t = 0; t < CT; ++t) {
                        const int f = 64 * t + 16 * w + 4 * g;
                        const float4 qq = load4_f32<S>(sm.q + (16 * j + n) * ST + f);
                        const float qv[4] = {qq.x, qq.y, qq.z, qq.w};
                        float z[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) z[i] = qv[i] + gam[t][i] * ((hqT[j][t][i] - mu) * r) + bet[t][i];
                        *reinterpret_cast<float4*>(Zu + (size_t)(c0 + 16 * j + n) * D + f) =
                            make_float4(z[0], z[1], z[2], z[3]);
                    }
                }
            }
        }

        // ======== the next chunk into the stage ========
        if (c1 < N) {
            __syncthreads();                       // every wave is done with this block's stage
            if constexpr (!G::PREFETCH) mid_load<D, NG, S, G::PPT>(pf, pe, c1, N, tid, Qu, Ku, Vu, etau, eta_const);
            const int bc1 = block_rows(c1);
            mid_store<D, NG, S, G::PPT>(sm, pf, pe, tid, bc1);
            if constexpr (G::PREFETCH)
                if (c1 + bc1 < N) mid_load<D, NG, S, G::PPT>(pf, pe, c1 + bc1, N, tid, Qu, Ku, Vu, etau, eta_const);
            __syncthreads();
        }
        c0 = c1;
    }

    // W_end = W0 + (accumulated change) for the LN kind (W0 - mean formed with the
    // rounding it had at the start, so an unmoved state comes back bit for bit);
    // every entry is read and written by one lane, so W_end may be W0.
    float* Wu = Wend + unit * (size_t)D * D;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t o = (size_t)(16 * r + 4 * g + i) * D + 64 * t + 16 * w + n;
                float v = Wacc[r][t][i];
                if constexpr (KIND == 1) {
                    const float w0 = W0u[o];
                    v = w0 + (v - (w0 - row_mean(16 * r + 4 * g + i)));
                }
                Wu[o] = v;
            }
}

template <int D, int NG, int KIND, typename S, bool BIG, int APPLY = APPLY_DUAL>
hipError_t launch_one(const LinearArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((midb_linear_kernel<D, NG, KIND, S, BIG, APPLY>), dim3(a.B * a.H), dim3(MB_THREADS), 0, stream,
                       a.H,
                       a.N, a.b, static_cast<const S*>(a.Q), static_cast<const S*>(a.K), static_cast<const S*>(a.V),
                       a.eta, a.eta_const, a.W0, a.gamma, a.beta, a.eps, a.Z, a.W_end);
    return hipGetLastError();
}

template <int D, int NG, typename S>
hipError_t launch_kind(const LinearArgs& a, hipStream_t stream)
{
    return a.kind == 1 ? launch_one<D, NG, 1, S, false>(a, stream) : launch_one<D, NG, 0, S, false>(a, stream);
}

template <int D, typename S>
hipError_t launch_groups(const LinearArgs& a, hipStream_t stream)
{
    const int ng = (a.b + 15) / 16;
    if (ng == 1) return launch_kind<D, 1, S>(a, stream);
    if (ng == 2) return launch_kind<D, 2, S>(a, stream);
    if (ng == 3) return launch_kind<D, 3, S>(a, stream);
    return launch_kind<D, 4, S>(a, stream);
}

template <int APPLY>
hipError_t launch_blocks(const LinearArgs& a, hipStream_t stream)
{
    if (a.d == 128)
        return a.dtype == 1 ? launch_one<128, 4, 0, uint16_t, true, APPLY>(a, stream)
                            : launch_one<128, 4, 0, float, true, APPLY>(a, stream);
    return a.dtype == 1 ? launch_one<64, 4, 0, uint16_t, true, APPLY>(a, stream)
                        : launch_one<64, 4, 0, float, true, APPLY>(a, stream);
}

}  // namespace

hipError_t launch_midb_linear_blocks(const LinearArgs& a, int outputs, hipStream_t stream)
{
    if (outputs == LC_OUT_BEFORE) return launch_blocks<APPLY_BEFORE>(a, stream);
    if (outputs == LC_OUT_AFTER) return launch_blocks<APPLY_AFTER>(a, stream);
    return launch_blocks<APPLY_DUAL>(a, stream);
}

hipError_t launch_midb_linear(const LinearArgs& a, hipStream_t stream)
{
    if (a.d == 128)
        return a.dtype == 1 ? launch_groups<128, uint16_t>(a, stream) : launch_groups<128, float>(a, stream);
    return a.dtype == 1 ? launch_groups<64, uint16_t>(a, stream) : launch_groups<64, float>(a, stream);
}

}  // namespace ttt
