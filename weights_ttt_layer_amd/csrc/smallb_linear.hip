// smallb_linear.hip -- TTT-Linear forward (plain and LayerNorm+residual inner
// model) for small mini-batches, d = 64, 1 <= b <= 16.
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
//  * One workgroup (4 waves, 256 lanes) per (sequence, head) unit. Wave w owns
//    the state columns [16w, 16w+16) as four 16x16 fp32 MFMA accumulator tiles;
//    W never leaves the registers between the first load of W0 and the final
//    store of W_end (the pages' "weight update in SRAM" idea, page "How to
//    Master Test-Time Training for Infinite Context LLMs").
//  * The accumulator layout of W is used directly as the B operand of the next
//    K W_c and Q W_c products: the k index of a 16x16x32 B operand is taken in
//    the permuted order (tile 2p rows 4g..4g+3, then tile 2p+1 rows 4g..4g+3)
//    and the A operands (K, Q rows) are read from LDS in the same order.
//  * The gradient Gt, produced in the C layout of H_K, is directly the B
//    operand of both K^T Gt (state update) and tril(QK^T) Gt.
//  * S^T = K Q^T is computed instead of Q K^T because its C layout is exactly
//    the A operand layout of the 16x16x16 product tril(S) Gt.
//  * fp32 operands (W, Gt, S) are split into bf16 terms (2 for bf16 token
//    streams, 3 for fp32 streams); fp32 token streams use 3 terms as well.
//  * Q/K/V/eta chunks are prefetched into registers one chunk ahead and staged
//    through double-buffered, row-padded LDS tiles.
//  * LayerNorm statistics are row sums over the 64 columns: a 16-lane DPP
//    reduction inside each wave, then a 4-wave exchange through LDS.
#include "device_common.h"
#include "kernels.h"

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int ROWS = 16;
constexpr int THREADS = 256;

template <typename S>
struct Stor;
template <>
struct Stor<uint16_t> {  // bf16 bit patterns
    static constexpr int TERMS = 1;
    static constexpr int STRIDE = D + 8;              // elements per LDS row (144 B)
    static constexpr int PIECES = D * 2 / 16;          // 16-byte pieces per row
    __device__ static float f(uint16_t x) { return __builtin_bit_cast(float, (uint32_t)x << 16); }
};
template <>
struct Stor<float> {
    static constexpr int TERMS = 3;
    static constexpr int STRIDE = D + 4;              // 272 B
    static constexpr int PIECES = D * 4 / 16;
    __device__ static float f(float x) { return x; }
};

// Eight consecutive-in-k operand elements given as two groups of four, p0[0..3]
// and p1[0..3], as TERMS bf16x8 terms.
template <typename S, int T>
__device__ __forceinline__ void load_a8(const S* p0, const S* p1, bf16x8 (&out)[T])
{
    if constexpr (sizeof(S) == 2) {
        static_assert(T == 1, "bf16 streams are exact in one term");
        uint2 a = *reinterpret_cast<const uint2*>(p0);
        uint2 b = *reinterpret_cast<const uint2*>(p1);
        uint4 v = make_uint4(a.x, a.y, b.x, b.y);
        out[0] = __builtin_bit_cast(bf16x8, v);
    } else {
        float4 a = *reinterpret_cast<const float4*>(p0);
        float4 b = *reinterpret_cast<const float4*>(p1);
        float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            __bf16 t[T];
            split_terms<T>(x[j], t);
#pragma unroll
            for (int s = 0; s < T; ++s) out[s][j] = t[s];
        }
    }
}

// Four operand elements x[0..3] (fp32 values) as T bf16x4 terms.
template <int T>
__device__ __forceinline__ void terms4(const float (&x)[4], bf16x4 (&out)[T])
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        __bf16 t[T];
        split_terms<T>(x[j], t);
#pragma unroll
        for (int s = 0; s < T; ++s) out[s][j] = bf16_bits(t[s]);
    }
}

template <typename S>
struct alignas(16) Stage {
    S q[ROWS * Stor<S>::STRIDE];
    S k[ROWS * Stor<S>::STRIDE];
    S v[ROWS * Stor<S>::STRIDE];
    float eta[ROWS];
};

template <typename S>
struct alignas(16) Smem {
    Stage<S> st[2];
    float red[3][4][ROWS][2];   // [exchange][wave][row][quantity]
};


template <typename S>
struct Pieces {
    static constexpr int PIECES = Stor<S>::PIECES;
    static constexpr int ELEMS_PER_PIECE = 16 / sizeof(S);
    static constexpr int TOTAL = 3 * ROWS * PIECES;
};

// Issue the global loads of chunk c (rows past the sequence end read as zero).
template <typename S, int PPT>
__device__ __forceinline__ void load_chunk(uint4 (&pf)[PPT], float& pe, int c, int b, int N, int tid,
                                           const S* Qu, const S* Ku, const S* Vu,
                                           const float* etau, float eta_const)
{
    using P = Pieces<S>;
    const int c0 = c * b;
    const int bc = min(b, N - c0);
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int idx = tid + k * THREADS;
        pf[k] = make_uint4(0, 0, 0, 0);
        if (idx < P::TOTAL) {
            const int tensor = idx / (ROWS * P::PIECES);
            const int rem = idx - tensor * (ROWS * P::PIECES);
            const int row = rem / P::PIECES;
            const int piece = rem - row * P::PIECES;
            const S* src = tensor == 0 ? Qu : (tensor == 1 ? Ku : Vu);
            if (row < bc)
                pf[k] = *reinterpret_cast<const uint4*>(src + (size_t)(c0 + row) * D +
                                                         piece * P::ELEMS_PER_PIECE);
        }
    }
    if (tid < ROWS) pe = tid < bc ? (etau ? etau[c0 + tid] : eta_const) : 0.f;
}

template <typename S, int PPT>
__device__ __forceinline__ void store_chunk(Stage<S>& st, const uint4 (&pf)[PPT], float pe, int tid)
{
    using P = Pieces<S>;
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int idx = tid + k * THREADS;
        if (idx < P::TOTAL) {
            const int tensor = idx / (ROWS * P::PIECES);
            const int rem = idx - tensor * (ROWS * P::PIECES);
            const int row = rem / P::PIECES;
            const int piece = rem - row * P::PIECES;
            S* dst = tensor == 0 ? st.q : (tensor == 1 ? st.k : st.v);
            *reinterpret_cast<uint4*>(dst + row * Stor<S>::STRIDE + piece * P::ELEMS_PER_PIECE) = pf[k];
        }
    }
    if (tid < ROWS) st.eta[tid] = pe;
}

template <int KIND, typename S>
__global__ void __launch_bounds__(THREADS)
smallb_linear_kernel(int H, int N, int b, const S* __restrict__ Qg, const S* __restrict__ Kg,
                     const S* __restrict__ Vg, const float* __restrict__ etag, float eta_const,
                     const float* __restrict__ W0, const float* __restrict__ gamma,
                     const float* __restrict__ beta, float eps, float* __restrict__ Zg,
                     float* __restrict__ Wend)
{
    constexpr int TIN = Stor<S>::TERMS;               // terms of a token-stream operand
    constexpr int TS = (TIN == 1) ? 2 : 3;            // terms of an fp32 state operand
    constexpr int STRIDE = Stor<S>::STRIDE;
    constexpr int PPT = (Pieces<S>::TOTAL + THREADS - 1) / THREADS;

    __shared__ Smem<S> sm;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int n = lane & 15;
    const int col = 16 * w + n;

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
    float gam = 0.f, bet = 0.f;
    if constexpr (KIND == 1) {
        gam = gamma[h * D + col];
        bet = beta[h * D + col];
    }

    const int nchunks = (N + b - 1) / b;

    // ---- chunk prefetch: registers -> LDS ----
    uint4 pf[PPT];
    float pe = 0.f;
    if (nchunks > 0) {
        load_chunk<S, PPT>(pf, pe, 0, b, N, tid, Qu, Ku, Vu, etau, eta_const);
        store_chunk<S, PPT>(sm.st[0], pf, pe, tid);
    }

    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        const int c0 = c * b;
        const int bc = min(b, N - c0);
        if (c + 1 < nchunks) load_chunk<S, PPT>(pf, pe, c + 1, b, N, tid, Qu, Ku, Vu, etau, eta_const);
        __syncthreads();
        const Stage<S>& st = sm.st[buf];

        // ---- W_c as B operand terms (permuted k order) ----
        bf16x8 Wb[2][TS];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = j < 4 ? Wacc[2 * p][j] : Wacc[2 * p + 1][j - 4];
                __bf16 t[TS];
                split_terms<TS>(x, t);
#pragma unroll
                for (int s = 0; s < TS; ++s) Wb[p][s][j] = t[s];
            }

        // ---- H_K = K W_c, H_Q = Q W_c (row n of the A operand is token n) ----
        f32x4 hk = {0.f, 0.f, 0.f, 0.f};
        f32x4 hq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            bf16x8 ka[TIN], qa[TIN];
            const int o0 = n * STRIDE + 32 * p + 4 * g;
            load_a8<S, TIN>(st.k + o0, st.k + o0 + 16, ka);
            load_a8<S, TIN>(st.q + o0, st.q + o0 + 16, qa);
            hk = mma32_terms<TIN, TS>(hk, ka, Wb[p]);
            hq = mma32_terms<TIN, TS>(hq, qa, Wb[p]);
        }

        // ---- S^T = K Q^T: lane (g, n) gets S[n][4g+i] = q_n . k_{4g+i} ----
        f32x4 sT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            bf16x8 ka[TIN], qb[TIN];
            const int o = n * STRIDE + 32 * p + 8 * g;
            load_a8<S, TIN>(st.k + o, st.k + o + 4, ka);
            load_a8<S, TIN>(st.q + o, st.q + o + 4, qb);
            sT = mma32_terms<TIN, TIN>(sT, ka, qb);
        }

        // ---- per-element values in the C layout: row 4g+i, column col ----
        float vv[4], et[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            vv[i] = Stor<S>::f(st.v[(4 * g + i) * STRIDE + col]);
            et[i] = st.eta[4 * g + i];
        }

        float gt[4];
        if constexpr (KIND == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) gt[i] = et[i] * 2.f * (hk[i] - vv[i]);
        } else {
            // LayerNorm forward statistics of H_K rows
            float s1[4], s2[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s1[i] = row16_sum(hk[i]);
                s2[i] = row16_sum(hk[i] * hk[i]);
            }
            if (n == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sm.red[0][w][4 * g + i][0] = s1[i];
                    sm.red[0][w][4 * g + i][1] = s2[i];
                }
            }
            __syncthreads();
            float mu[4], rs[4], xh[4], dxh[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float a = 0.f, q2 = 0.f;
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) {
                    a += sm.red[0][ww][4 * g + i][0];
                    q2 += sm.red[0][ww][4 * g + i][1];
                }
                mu[i] = a * (1.f / D);
                const float var = fmaxf(q2 * (1.f / D) - mu[i] * mu[i], 0.f);
                rs[i] = 1.f / sqrtf(var + eps);
                xh[i] = (hk[i] - mu[i]) * rs[i];
                const float kk = Stor<S>::f(st.k[(4 * g + i) * STRIDE + col]);
                const float e = kk + gam * xh[i] + bet - vv[i];
                dxh[i] = 2.f * e * gam;
            }
            // LayerNorm backward: means of dxh and dxh*xh over the row
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s1[i] = row16_sum(dxh[i]);
                s2[i] = row16_sum(dxh[i] * xh[i]);
            }
            if (n == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sm.red[1][w][4 * g + i][0] = s1[i];
                    sm.red[1][w][4 * g + i][1] = s2[i];
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float m1 = 0.f, m2 = 0.f;
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) {
                    m1 += sm.red[1][ww][4 * g + i][0];
                    m2 += sm.red[1][ww][4 * g + i][1];
                }
                const float gg = rs[i] * (dxh[i] - m1 * (1.f / D) - xh[i] * (m2 * (1.f / D)));
                gt[i] = et[i] * gg;
            }
        }
        // padded rows contribute nothing (guards eps = 0 on all-zero rows)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * g + i >= bc) gt[i] = 0.f;

        // ---- -Gt as B operand terms (k index = token 4g+i) ----
        bf16x4 gb[TS];
        {
            float x[4] = {-gt[0], -gt[1], -gt[2], -gt[3]};
            terms4<TS>(x, gb);
        }

        // ---- H_Q -= tril(S) Gt  (A = S with row n, k = 4g+i) ----
        {
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (4 * g + i <= n) ? sT[i] : 0.f;
            bf16x4 sa[TS];
            terms4<TS>(x, sa);
            hq = mma16_terms<TS, TS>(hq, sa, gb);
        }

        // ---- W_{c+1} = W_c - K^T Gt  (A = K^T tile r: row m = feature, k = token) ----
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = Stor<S>::f(st.k[(4 * g + j) * STRIDE + 16 * r + n]);
            bf16x4 kt[TIN];
            terms4<TIN>(x, kt);
            Wacc[r] = mma16_terms<TIN, TS>(Wacc[r], kt, gb);
        }

        // ---- output ----
        float z[4];
        if constexpr (KIND == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) z[i] = hq[i];
        } else {
            float s1[4], s2[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s1[i] = row16_sum(hq[i]);
                s2[i] = row16_sum(hq[i] * hq[i]);
            }
            if (n == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sm.red[2][w][4 * g + i][0] = s1[i];
                    sm.red[2][w][4 * g + i][1] = s2[i];
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float a = 0.f, q2 = 0.f;
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) {
                    a += sm.red[2][ww][4 * g + i][0];
                    q2 += sm.red[2][ww][4 * g + i][1];
                }
                const float mu = a * (1.f / D);
                const float var = fmaxf(q2 * (1.f / D) - mu * mu, 0.f);
                const float rs = 1.f / sqrtf(var + eps);
                const float qq = Stor<S>::f(st.q[(4 * g + i) * STRIDE + col]);
                z[i] = qq + gam * ((hq[i] - mu) * rs) + bet;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * g + i < bc) Zu[(size_t)(c0 + 4 * g + i) * D + col] = z[i];

        if (c + 1 < nchunks) store_chunk<S, PPT>(sm.st[buf ^ 1], pf, pe, tid);
    }

    float* Wu = Wend + unit * (size_t)D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) Wu[(16 * r + 4 * g + i) * D + col] = Wacc[r][i];
}

template <int KIND, typename S>
hipError_t launch_typed(const LinearArgs& a, hipStream_t stream)
{
    const int units = a.B * a.H;
    hipLaunchKernelGGL((smallb_linear_kernel<KIND, S>), dim3(units), dim3(THREADS), 0, stream, a.H,
                       a.N, a.b, static_cast<const S*>(a.Q), static_cast<const S*>(a.K),
                       static_cast<const S*>(a.V), a.eta, a.eta_const, a.W0, a.gamma, a.beta,
                       a.eps, a.Z, a.W_end);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_smallb_linear(const LinearArgs& a, hipStream_t stream)
{
    if (a.dtype == 1)
        return a.kind == 1 ? launch_typed<1, uint16_t>(a, stream) : launch_typed<0, uint16_t>(a, stream);
    return a.kind == 1 ? launch_typed<1, float>(a, stream) : launch_typed<0, float>(a, stream);
}

}  // namespace ttt
