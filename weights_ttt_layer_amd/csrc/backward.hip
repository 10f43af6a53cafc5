// backward.hip -- backward of TTT-Linear (plain and LayerNorm + residual inner
// model) through the mini-batch dual form, d = 64, 1 <= b <= 16: the gradients
// of a scalar objective with respect to Q, K, V, eta, W0 (and gamma, beta)
// given its gradients dZ and dW_end. Page "Test-Time Training: Linear
// Complexity Beyond Attention" (section "1. The Self-Supervised Inner-Loop
// Task") trains the outer parameters by backpropagation through the inner
// loop; this is that backpropagation for the chunked form of section "4.
// Mini-Batch Parallelism (Dual Formulation)". Per chunk (rows t, s; s <= t):
//     h_s = k_s W_c,  g_s = d l_s / d h_s,  a_ts = q_t . k_s
//     hq_t = q_t W_c - sum_{s<=t} a_ts eta_s g_s,   z_t = hq_t  or  q_t + LN(hq_t)
//     W_{c+1} = W_c - sum_s eta_s k_s^T g_s
//
// One workgroup (four waves) per (sequence, head) unit, two passes:
//  1. the chunk-start states W_c are recomputed and written to the workspace;
//  2. the chunks are visited in reverse. dW (the gradient with respect to the
//     state at the current chunk boundary) stays in LDS; each chunk first uses
//     it as d/dW_{c+1}, then adds the chunk's own terms to make it d/dW_c.
// Every matrix product runs on the fp32 matrix cores (v_mfma_f32_16x16x4f32,
// exact fp32 products) over operands staged in LDS; each wave owns one
// 16-column tile of a 16 x 64 result (or one 16-row band of a 64 x 64 one).
// The row-wise steps (LayerNorm statistics and their derivatives) give every
// token row to one DPP row of 16 lanes, four entries per lane.
#include "device_common.h"
#include "kernels.h"

namespace ttt {
namespace {

constexpr int BD = 64;       // head dim
constexpr int BR = 16;       // rows of a chunk tile (b <= 16)
constexpr int BT = 256;      // threads per workgroup
constexpr int LS = 68;       // LDS row stride (floats) of 64-wide tiles
constexpr int SS = 20;       // LDS row stride of 16-wide tiles

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc +/- sum_k A(i, k) B(k, j) for a 16 x 16 tile, k < KD (a multiple of 16).
// The accessors return four consecutive k: a(i, k) = A(i, k .. k+3),
// b(k, j) = B(k .. k+3, j). Lane l supplies row / column l % 16 at
// k = k0 + 4 (l / 16) + u to product u, so an operand stored with k contiguous is
// one 16-byte read. acc and the result are in the C layout (lane l: rows
// 4 (l / 16) + r, column l % 16). One accumulation chain: an fp32 16x16x4
// product keeps the matrix pipe busy for as long as its result takes, so
// independent chains would add no throughput, only moves and sums.
template <int KD, bool SUB = false, class FA, class FB>
__device__ __forceinline__ f32x4 tile_mm(f32x4 acc, FA a, FB b, int lane)
{
    const int i = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < KD; k0 += 16) {
        float4 av = a(i, k0 + 4 * kq);
        const float4 bv = b(k0 + 4 * kq, i);
        if constexpr (SUB) av = make_float4(-av.x, -av.y, -av.z, -av.w);
        acc = mfma4(av.x, bv.x, acc);
        acc = mfma4(av.y, bv.y, acc);
        acc = mfma4(av.z, bv.z, acc);
        acc = mfma4(av.w, bv.w, acc);
    }
    return acc;
}

constexpr f32x4 ZERO4 = {0.f, 0.f, 0.f, 0.f};

// Operand accessors: rows of a row-major tile (k contiguous), or a column of
// one (k strided).
#define ROW4(M, i, k) (*reinterpret_cast<const float4*>(&(M)[i][k]))
#define COL4(M, k, j) make_float4((M)[k][j], (M)[(k) + 1][j], (M)[(k) + 2][j], (M)[(k) + 3][j])

// C-layout tile stored transposed (row-major m^T)
__device__ __forceinline__ void st_tile_t(float* m, int stride, int r0, int c0, const f32x4& v, int lane)
{
    const int j = c0 + (lane & 15), i0 = r0 + 4 * (lane >> 4);
    *reinterpret_cast<float4*>(&m[j * stride + i0]) = make_float4(v[0], v[1], v[2], v[3]);
}

// C-layout tile <-> LDS (row-major, `stride` floats per row), rows r0.., cols c0..
__device__ __forceinline__ f32x4 ld_tile(const float* m, int stride, int r0, int c0, int lane)
{
    const int j = c0 + (lane & 15), i0 = r0 + 4 * (lane >> 4);
    f32x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = m[(i0 + r) * stride + j];
    return v;
}

__device__ __forceinline__ void st_tile(float* m, int stride, int r0, int c0, const f32x4& v, int lane)
{
    const int j = c0 + (lane & 15), i0 = r0 + 4 * (lane >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) m[(i0 + r) * stride + j] = v[r];
}

struct alignas(16) BwdSmem {
    float W[BD][LS];     // W_c (pass 2) / the running state (pass 1)
    float WT[BD][LS];    // its transpose
    float dW[BD][LS];    // gradient with respect to the state at the chunk boundary
    float dWT[BD][LS];   // its transpose
    float K[BR][LS], Q[BR][LS], V[BR][LS], dZ[BR][LS];
    float H[BR][LS];     // K W_c
    float HQ[BR][LS];    // Q W_c - A G
    float KD[BR][LS];    // K dW_{c+1}
    float GD[BR][LS];    // G dW_{c+1}^T
    float G[BR][LS];     // g_s (pass 1: eta_s g_s)
    float dG[BR][LS];
    float dHq[BR][LS];
    float dQ[BR][LS], dK[BR][LS], dV[BR][LS];
    float dh[BR][LS];
    float dKd[BR][LS];   // direct terms of dK from the preactivation-gradient backward
    float S[BR][SS];     // a_ts = q_t . k_s
    float P[BR][SS];     // dhq_t . g_s
    float DA[BR][SS];    // d a_ts (causal part)
    float C2[BR][SS];    // d eta_s contributions of the causal term, per t
    alignas(16) float eta[BR];
    alignas(16) float deta[BR];
    float red[2][BR][BD];
};

template <typename S>
__device__ __forceinline__ float4 load4(const S* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p)
{
    return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<uint16_t>(const uint16_t* p)
{
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__builtin_bit_cast(float, u.x << 16), __builtin_bit_cast(float, u.x & 0xFFFF0000u),
                       __builtin_bit_cast(float, u.y << 16), __builtin_bit_cast(float, u.y & 0xFFFF0000u));
}

__device__ __forceinline__ void put4(float* row, int j0, float4 v)
{
    *reinterpret_cast<float4*>(row + j0) = v;
}
__device__ __forceinline__ float4 get4(const float* row, int j0) { return *reinterpret_cast<const float4*>(row + j0); }

// Row-wise LayerNorm pieces: the 64 entries of a row sit in one DPP row of 16
// lanes, four per lane.
struct LnRow {
    float c[4], xh[4], r;
};

__device__ __forceinline__ LnRow ln_stats(const float (&h)[4], float eps)
{
    LnRow s;
    const float mu = row16_sum(h[0] + h[1] + h[2] + h[3]) * (1.f / BD);
#pragma unroll
    for (int e = 0; e < 4; ++e) s.c[e] = h[e] - mu;
    const float var = row16_sum(s.c[0] * s.c[0] + s.c[1] * s.c[1] + s.c[2] * s.c[2] + s.c[3] * s.c[3]) * (1.f / BD);
    s.r = 1.f / sqrtf(var + eps);
#pragma unroll
    for (int e = 0; e < 4; ++e) s.xh[e] = s.c[e] * s.r;
    return s;
}

// dh = r (gx - mean(gx) - xhat mean(gx xhat)), gx = gamma dy
__device__ __forceinline__ void ln_bwd(const LnRow& s, const float (&gam)[4], const float (&dy)[4], float (&dh)[4])
{
    float gx[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) gx[e] = gam[e] * dy[e];
    const float m1 = row16_sum(gx[0] + gx[1] + gx[2] + gx[3]) * (1.f / BD);
    const float m2 = row16_sum(gx[0] * s.xh[0] + gx[1] * s.xh[1] + gx[2] * s.xh[2] + gx[3] * s.xh[3]) * (1.f / BD);
#pragma unroll
    for (int e = 0; e < 4; ++e) dh[e] = s.r * (gx[e] - m1 - s.xh[e] * m2);
}

__device__ __forceinline__ void to4(float4 v, float (&a)[4]) { a[0] = v.x, a[1] = v.y, a[2] = v.z, a[3] = v.w; }
__device__ __forceinline__ float4 of4(const float (&a)[4]) { return make_float4(a[0], a[1], a[2], a[3]); }

// g = d ||f(k; W) - v||^2 / dh at h = k W (row r of sm.H), for KIND 0 (plain) or 1 (LN).
template <int KIND>
__device__ __forceinline__ void preact_grad(const float (&h)[4], const float (&k)[4], const float (&v)[4],
                                            const float (&gam)[4], const float (&bet)[4], float eps,
                                            float (&g)[4])
{
    if constexpr (KIND == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) g[e] = 2.f * (h[e] - v[e]);
    } else {
        const LnRow s = ln_stats(h, eps);
        float dy[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) dy[e] = 2.f * (k[e] + gam[e] * s.xh[e] + bet[e] - v[e]);
        ln_bwd(s, gam, dy, g);
    }
}

template <int KIND, typename S>
__global__ void __launch_bounds__(BT)
bwd_linear_kernel(int H, int N, int b, const S* __restrict__ Qg, const S* __restrict__ Kg,
                  const S* __restrict__ Vg, const float* __restrict__ etag, float eta_const,
                  const float* __restrict__ W0, const float* __restrict__ gamma, const float* __restrict__ beta,
                  float eps, const float* __restrict__ dZg, const float* __restrict__ dWend,
                  float* __restrict__ dQg, float* __restrict__ dKg, float* __restrict__ dVg,
                  float* __restrict__ detag, float* __restrict__ dW0g, float* __restrict__ ckpt,
                  float* __restrict__ gbpart)
{
    __shared__ BwdSmem sm;
    const int unit = blockIdx.x, head = unit % H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = tid >> 4, j0 = (tid & 15) * 4;          // row-phase layout
    const int C = (N + b - 1) / b;
    const size_t tok0 = (size_t)unit * N;
    float* ck = ckpt + (size_t)unit * C * BD * BD;

    float gam[4] = {0.f, 0.f, 0.f, 0.f}, bet[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KIND == 1) {
        to4(get4(gamma + head * BD, j0), gam);
        to4(get4(beta + head * BD, j0), bet);
    }
    float pg[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f};   // dgamma, dbeta partials

    // this thread's four entries of row r of a token stream (zero past n)
    auto fetch_row = [&](const S* src, int t0, int n) {
        return r < n ? load4(src + (tok0 + t0 + r) * BD + j0) : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    auto fetch_eta = [&](int t0, int n) {
        return tid < n ? (etag ? etag[tok0 + t0 + tid] : eta_const) : 0.f;
    };
    // this thread's four float4 of a 64 x 64 fp32 matrix
    auto fetch_mat = [&](const float* src, float4 (&m4)[4]) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int i = tid + BT * m, row = i >> 4, col = (i & 15) * 4;
            m4[m] = src ? get4(src + row * BD, col) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    // ... into LDS, with its transpose
    auto put_mat = [&](float (*M)[LS], float (*MT)[LS], const float4 (&m4)[4]) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int i = tid + BT * m, row = i >> 4, col = (i & 15) * 4;
            put4(M[row], col, m4[m]);
            MT[col][row] = m4[m].x;
            MT[col + 1][row] = m4[m].y;
            MT[col + 2][row] = m4[m].z;
            MT[col + 3][row] = m4[m].w;
        }
    };
    // Operands of the next chunk are requested while the current one is
    // processed; they wait in these registers.
    float4 pk, pq, pv, pz, pw[4];
    float pe;

    // ---------------- pass 1: chunk-start states ----------------
    fetch_mat(W0 + (size_t)unit * BD * BD, pw);
    if constexpr (KIND == 1) {
        // LN kind: the recomputed states carry each row's mean over the output
        // features removed. The forward is unchanged by it (LayerNorm ignores a
        // constant added to a whole row, and the LayerNorm gradient of every
        // token sums to zero over the features, so the update never moves the
        // row means), and so is every gradient: the products with W^T
        // (dH_Q W^T, dh W^T) take row-gradients that also sum to zero over the
        // features. Without the means those products do not cancel a large
        // common part in fp32. A row's 64 entries sit in one 16-lane DPP row.
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float mean = row16_sum((pw[m].x + pw[m].y) + (pw[m].z + pw[m].w)) * (1.f / BD);
            pw[m] = make_float4(pw[m].x - mean, pw[m].y - mean, pw[m].z - mean, pw[m].w - mean);
        }
    }
    put_mat(sm.W, sm.WT, pw);
    pk = fetch_row(Kg, 0, min(b, N));
    pv = fetch_row(Vg, 0, min(b, N));
    pe = fetch_eta(0, min(b, N));
    for (int c = 0; c < C; ++c) {
        const int t0 = c * b, n = min(b, N - t0);
        put4(sm.K[r], j0, pk);
        put4(sm.V[r], j0, pv);
        if (tid < BR) sm.eta[tid] = pe;
        if (c + 1 < C) {
            const int t1 = t0 + b, n1 = min(b, N - t1);
            pk = fetch_row(Kg, t1, n1);
            pv = fetch_row(Vg, t1, n1);
            pe = fetch_eta(t1, n1);
        }
        __syncthreads();
        for (int i = tid; i < BD * BD / 4; i += BT) {
            const int row = i >> 4, col = (i & 15) * 4;
            *reinterpret_cast<float4*>(ck + (size_t)c * BD * BD + row * BD + col) = get4(sm.W[row], col);
        }
        // H = K W
        {
            const f32x4 t = tile_mm<BD>(ZERO4, [&](int i, int k) { return ROW4(sm.K, i, k); },
                                        [&](int k, int j) { return ROW4(sm.WT, 16 * w + j, k); }, lane);
            st_tile(&sm.H[0][0], LS, 0, 16 * w, t, lane);
        }
        __syncthreads();
        {
            float h[4], k[4], v[4], g[4];
            to4(get4(sm.H[r], j0), h);
            to4(get4(sm.K[r], j0), k);
            to4(get4(sm.V[r], j0), v);
            preact_grad<KIND>(h, k, v, gam, bet, eps, g);
            const float e = sm.eta[r];
            put4(sm.G[r], j0, r < n ? make_float4(e * g[0], e * g[1], e * g[2], e * g[3])
                                    : make_float4(0.f, 0.f, 0.f, 0.f));
        }
        __syncthreads();
        // W -= K^T (eta G): wave w updates rows 16w .. 16w + 15
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            f32x4 acc = ld_tile(&sm.W[0][0], LS, 16 * w, 16 * tj, lane);
            acc = tile_mm<BR, true>(acc, [&](int i, int k) { return COL4(sm.K, k, 16 * w + i); },
                               [&](int k, int j) { return COL4(sm.G, k, 16 * tj + j); }, lane);
            st_tile(&sm.W[0][0], LS, 16 * w, 16 * tj, acc, lane);
            st_tile_t(&sm.WT[0][0], LS, 16 * w, 16 * tj, acc, lane);
        }
        __syncthreads();
    }
    // the checkpoints are read back by other waves of this workgroup
    __threadfence();
    __syncthreads();

    // ---------------- pass 2: reverse sweep ----------------
    fetch_mat(dWend ? dWend + (size_t)unit * BD * BD : nullptr, pw);
    put_mat(sm.dW, sm.dWT, pw);
    auto fetch2 = [&](int c) {
        const int t0 = c * b, n = min(b, N - t0);
        pk = fetch_row(Kg, t0, n);
        pq = fetch_row(Qg, t0, n);
        pv = fetch_row(Vg, t0, n);
        pz = r < n ? get4(dZg + (tok0 + t0 + r) * BD, j0) : make_float4(0.f, 0.f, 0.f, 0.f);
        pe = fetch_eta(t0, n);
        fetch_mat(ck + (size_t)c * BD * BD, pw);
    };
    fetch2(C - 1);
    for (int c = C - 1; c >= 0; --c) {
        const int t0 = c * b, n = min(b, N - t0);
        // A: operands of the chunk (requested one chunk ahead)
        put4(sm.K[r], j0, pk);
        put4(sm.Q[r], j0, pq);
        put4(sm.V[r], j0, pv);
        put4(sm.dZ[r], j0, pz);
        if (tid < BR) sm.eta[tid] = pe;
        put_mat(sm.W, sm.WT, pw);
        if (c > 0) fetch2(c - 1);
        __syncthreads();
        // B: H = K W_c, HQ = Q W_c, KD = K dW_{c+1}, S = Q K^T
        {
            const int cw = 16 * w;
            const f32x4 th = tile_mm<BD>(ZERO4, [&](int i, int k) { return ROW4(sm.K, i, k); },
                                         [&](int k, int j) { return ROW4(sm.WT, cw + j, k); }, lane);
            const f32x4 tq = tile_mm<BD>(ZERO4, [&](int i, int k) { return ROW4(sm.Q, i, k); },
                                         [&](int k, int j) { return ROW4(sm.WT, cw + j, k); }, lane);
            const f32x4 tk = tile_mm<BD>(ZERO4, [&](int i, int k) { return ROW4(sm.K, i, k); },
                                         [&](int k, int j) { return ROW4(sm.dWT, cw + j, k); }, lane);
            st_tile(&sm.H[0][0], LS, 0, cw, th, lane);
            st_tile(&sm.HQ[0][0], LS, 0, cw, tq, lane);
            st_tile(&sm.KD[0][0], LS, 0, cw, tk, lane);
            if (w == 0)
                st_tile(&sm.S[0][0], SS, 0, 0,
                        tile_mm<BD>(ZERO4, [&](int i, int k) { return ROW4(sm.Q, i, k); },
                                    [&](int k, int j) { return ROW4(sm.K, j, k); }, lane), lane);
        }
        __syncthreads();
        // C: g_s at W_c
        {
            float h[4], k[4], v[4], g[4];
            to4(get4(sm.H[r], j0), h);
            to4(get4(sm.K[r], j0), k);
            to4(get4(sm.V[r], j0), v);
            preact_grad<KIND>(h, k, v, gam, bet, eps, g);
            put4(sm.G[r], j0, r < n ? of4(g) : make_float4(0.f, 0.f, 0.f, 0.f));
        }
        __syncthreads();
        // D: HQ -= A G (A_ts = a_ts eta_s, s <= t), GD = G dW_{c+1}^T
        {
            const int cw = 16 * w;
            f32x4 acc = ld_tile(&sm.HQ[0][0], LS, 0, cw, lane);
            acc = tile_mm<BR, true>(acc, 
                [&](int i, int k) {
                    const float4 s4 = ROW4(sm.S, i, k), e4 = *reinterpret_cast<const float4*>(&sm.eta[k]);
                    return make_float4(k <= i ? s4.x * e4.x : 0.f, k + 1 <= i ? s4.y * e4.y : 0.f,
                                       k + 2 <= i ? s4.z * e4.z : 0.f, k + 3 <= i ? s4.w * e4.w : 0.f);
                },
                [&](int k, int j) { return COL4(sm.G, k, cw + j); }, lane);
            st_tile(&sm.HQ[0][0], LS, 0, cw, acc, lane);
            st_tile(&sm.GD[0][0], LS, 0, cw,
                    tile_mm<BD>(ZERO4, [&](int i, int k) { return ROW4(sm.G, i, k); },
                                [&](int k, int j) { return ROW4(sm.dW, cw + j, k); }, lane), lane);
        }
        __syncthreads();
        // E: output stage, and the terms of W_{c+1} = W_c - sum_s eta_s k_s^T g_s
        {
            float dz[4], dhq[4], dq[4] = {0.f, 0.f, 0.f, 0.f};
            to4(get4(sm.dZ[r], j0), dz);
            if constexpr (KIND == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) dhq[e] = dz[e];
            } else {
                float hq[4];
                to4(get4(sm.HQ[r], j0), hq);
                const LnRow s = ln_stats(hq, eps);
                ln_bwd(s, gam, dz, dhq);
                if (r < n) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dq[e] = dz[e];
                        pg[e] += dz[e] * s.xh[e];
                        pb[e] += dz[e];
                    }
                }
            }
            float kd[4], gd[4], g[4];
            to4(get4(sm.KD[r], j0), kd);
            to4(get4(sm.GD[r], j0), gd);
            to4(get4(sm.G[r], j0), g);
            const float e = sm.eta[r];
            const float kdg = row16_sum(kd[0] * g[0] + kd[1] * g[1] + kd[2] * g[2] + kd[3] * g[3]);
            const bool live = r < n;
            put4(sm.dHq[r], j0, live ? of4(dhq) : make_float4(0.f, 0.f, 0.f, 0.f));
            put4(sm.dQ[r], j0, of4(dq));
            put4(sm.dG[r], j0, live ? make_float4(-e * kd[0], -e * kd[1], -e * kd[2], -e * kd[3])
                                    : make_float4(0.f, 0.f, 0.f, 0.f));
            put4(sm.dK[r], j0, live ? make_float4(-e * gd[0], -e * gd[1], -e * gd[2], -e * gd[3])
                                    : make_float4(0.f, 0.f, 0.f, 0.f));
            if ((tid & 15) == 0) sm.deta[r] = live ? -kdg : 0.f;
        }
        __syncthreads();
        // F: dQ += dHq W_c^T, dG -= A^T dHq, P = dHq G^T
        {
            const int cw = 16 * w;
            f32x4 acc = ld_tile(&sm.dQ[0][0], LS, 0, cw, lane);
            acc = tile_mm<BD>(acc, [&](int i, int k) { return ROW4(sm.dHq, i, k); },
                               [&](int k, int j) { return ROW4(sm.W, cw + j, k); }, lane);
            st_tile(&sm.dQ[0][0], LS, 0, cw, acc, lane);
            f32x4 ag = ld_tile(&sm.dG[0][0], LS, 0, cw, lane);
            ag = tile_mm<BR, true>(ag, 
                [&](int i, int k) {
                    const float4 s4 = COL4(sm.S, k, i);
                    const float e = sm.eta[i];
                    return make_float4(i <= k ? s4.x * e : 0.f, i <= k + 1 ? s4.y * e : 0.f,
                                       i <= k + 2 ? s4.z * e : 0.f, i <= k + 3 ? s4.w * e : 0.f);
                },
                [&](int k, int j) { return COL4(sm.dHq, k, cw + j); }, lane);
            st_tile(&sm.dG[0][0], LS, 0, cw, ag, lane);
            if (w == 0)
                st_tile(&sm.P[0][0], SS, 0, 0,
                        tile_mm<BD>(ZERO4, [&](int i, int k) { return ROW4(sm.dHq, i, k); },
                                    [&](int k, int j) { return ROW4(sm.G, j, k); }, lane), lane);
        }
        __syncthreads();
        // G: causal-term derivatives, d(a_ts eta_s) = -dhq_t . g_s, and, independent of
        // them, the backward of g = d l / d h: dh and the direct terms of dK, dV,
        // dgamma, dbeta
        {
            const int t = tid >> 4, s = tid & 15;
            const bool on = s <= t && t < n;
            const float dcoef = on ? -sm.P[t][s] : 0.f;
            sm.DA[t][s] = dcoef * sm.eta[s];
            sm.C2[t][s] = dcoef * sm.S[t][s];
        }
        {
            float dg[4], dh[4], dv[4], dkd[4] = {0.f, 0.f, 0.f, 0.f};
            to4(get4(sm.dG[r], j0), dg);
            if constexpr (KIND == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dh[e] = 2.f * dg[e];
                    dv[e] = -2.f * dg[e];
                }
            } else {
                float h[4], k[4], v[4];
                to4(get4(sm.H[r], j0), h);
                to4(get4(sm.K[r], j0), k);
                to4(get4(sm.V[r], j0), v);
                const LnRow s = ln_stats(h, eps);
                float dy[4], gx[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dy[e] = 2.f * (k[e] + gam[e] * s.xh[e] + bet[e] - v[e]);
                    gx[e] = gam[e] * dy[e];
                }
                const float m1 = row16_sum(gx[0] + gx[1] + gx[2] + gx[3]) * (1.f / BD);
                const float m2 =
                    row16_sum(gx[0] * s.xh[0] + gx[1] * s.xh[1] + gx[2] * s.xh[2] + gx[3] * s.xh[3]) * (1.f / BD);
                // through g = r (gx - m1 - xhat m2)
                float dr = row16_sum(dg[0] * (gx[0] - m1 - s.xh[0] * m2) + dg[1] * (gx[1] - m1 - s.xh[1] * m2) +
                                     dg[2] * (gx[2] - m1 - s.xh[2] * m2) + dg[3] * (gx[3] - m1 - s.xh[3] * m2));
                const float s1 = row16_sum(dg[0] + dg[1] + dg[2] + dg[3]);
                const float s2 = row16_sum(dg[0] * s.xh[0] + dg[1] * s.xh[1] + dg[2] * s.xh[2] + dg[3] * s.xh[3]);
                const float dm1 = -s.r * s1, dm2 = -s.r * s2;
                float dxh[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float dgx = s.r * dg[e] + dm1 * (1.f / BD) + dm2 * s.xh[e] * (1.f / BD);
                    dxh[e] = -s.r * dg[e] * m2 + dm2 * gx[e] * (1.f / BD);
                    // through gx = gamma dy and dy = 2 (k + gamma xhat + beta - v)
                    const float ddy = dgx * gam[e];
                    if (r < n) {
                        pg[e] += dgx * dy[e] + 2.f * ddy * s.xh[e];
                        pb[e] += 2.f * ddy;
                    }
                    dkd[e] = 2.f * ddy;
                    dxh[e] += 2.f * ddy * gam[e];
                    dv[e] = -2.f * ddy;
                }
                // through xhat = c r, r = (var + eps)^(-1/2), var = mean(c^2), c = h - mu
                dr += row16_sum(dxh[0] * s.c[0] + dxh[1] * s.c[1] + dxh[2] * s.c[2] + dxh[3] * s.c[3]);
                const float dvar = -0.5f * dr * s.r * s.r * s.r;
                float dc[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) dc[e] = dxh[e] * s.r + dvar * 2.f * s.c[e] * (1.f / BD);
                const float mdc = row16_sum(dc[0] + dc[1] + dc[2] + dc[3]) * (1.f / BD);
#pragma unroll
                for (int e = 0; e < 4; ++e) dh[e] = dc[e] - mdc;
            }
            const bool live = r < n;
            put4(sm.dKd[r], j0, of4(dkd));
            put4(sm.dV[r], j0, live ? of4(dv) : make_float4(0.f, 0.f, 0.f, 0.f));
            put4(sm.dh[r], j0, live ? of4(dh) : make_float4(0.f, 0.f, 0.f, 0.f));
        }
        __syncthreads();
        // H: dQ += DA K;  dK += DA^T Q + (direct terms) + dh W_c^T;
        //    dW += Q^T dHq + K^T dh  (wave w: rows 16w .. 16w + 15);  d eta_s += sum_t C2[t][s]
        {
            const int cw = 16 * w;
            f32x4 acc = ld_tile(&sm.dQ[0][0], LS, 0, cw, lane);
            acc = tile_mm<BR>(acc, [&](int i, int k) { return ROW4(sm.DA, i, k); },
                              [&](int k, int j) { return COL4(sm.K, k, cw + j); }, lane);
            st_tile(&sm.dQ[0][0], LS, 0, cw, acc, lane);
            f32x4 ak = ld_tile(&sm.dK[0][0], LS, 0, cw, lane) + ld_tile(&sm.dKd[0][0], LS, 0, cw, lane);
            ak = tile_mm<BR>(ak, [&](int i, int k) { return COL4(sm.DA, k, i); },
                             [&](int k, int j) { return COL4(sm.Q, k, cw + j); }, lane);
            ak = tile_mm<BD>(ak, [&](int i, int k) { return ROW4(sm.dh, i, k); },
                             [&](int k, int j) { return ROW4(sm.W, cw + j, k); }, lane);
            st_tile(&sm.dK[0][0], LS, 0, cw, ak, lane);
#pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                f32x4 aw = ld_tile(&sm.dW[0][0], LS, cw, 16 * tj, lane);
                aw = tile_mm<BR>(aw, [&](int i, int k) { return COL4(sm.Q, k, cw + i); },
                                 [&](int k, int j) { return COL4(sm.dHq, k, 16 * tj + j); }, lane);
                aw = tile_mm<BR>(aw, [&](int i, int k) { return COL4(sm.K, k, cw + i); },
                                 [&](int k, int j) { return COL4(sm.dh, k, 16 * tj + j); }, lane);
                st_tile(&sm.dW[0][0], LS, cw, 16 * tj, aw, lane);
                st_tile_t(&sm.dWT[0][0], LS, cw, 16 * tj, aw, lane);
            }
            if (tid < BR) {
                float a = 0.f;
#pragma unroll
                for (int t = 0; t < BR; ++t) a += sm.C2[t][tid];
                sm.deta[tid] += a;
            }
        }
        __syncthreads();
        // K: the chunk's gradients to HBM
        if (r < n) {
            const size_t o = (tok0 + t0 + r) * BD + j0;
            *reinterpret_cast<float4*>(dQg + o) = get4(sm.dQ[r], j0);
            *reinterpret_cast<float4*>(dKg + o) = get4(sm.dK[r], j0);
            *reinterpret_cast<float4*>(dVg + o) = get4(sm.dV[r], j0);
        }
        if (tid < n) detag[tok0 + t0 + tid] = sm.deta[tid];
        // the next chunk's loads touch none of the buffers read here
    }
    __syncthreads();
    for (int i = tid; i < BD * BD / 4; i += BT) {
        const int row = i >> 4, col = (i & 15) * 4;
        *reinterpret_cast<float4*>(dW0g + (size_t)unit * BD * BD + row * BD + col) = get4(sm.dW[row], col);
    }
    if constexpr (KIND == 1) {
        // per-unit dgamma, dbeta: sum the 16 row partials of each column
        put4(sm.red[0][r], j0, of4(pg));
        put4(sm.red[1][r], j0, of4(pb));
        __syncthreads();
        if (tid < 2 * BD) {
            const int which = tid >> 6, col = tid & 63;
            float a = 0.f;
#pragma unroll
            for (int t = 0; t < BR; ++t) a += sm.red[which][t][col];
            gbpart[((size_t)unit * 2 + which) * BD + col] = a;
        }
    }
}

// dgamma[h] = sum over sequences of the per-unit partials (fixed order)
__global__ void __launch_bounds__(2 * BD)
bwd_gamma_beta_kernel(int B, int H, const float* __restrict__ gbpart, float* __restrict__ dgamma,
                      float* __restrict__ dbeta)
{
    const int h = blockIdx.x, which = threadIdx.x >> 6, col = threadIdx.x & 63;
    float a = 0.f;
    for (int bi = 0; bi < B; ++bi) a += gbpart[(((size_t)bi * H + h) * 2 + which) * BD + col];
    (which == 0 ? dgamma : dbeta)[h * BD + col] = a;
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int b)
{
    const size_t units = (size_t)B * H, C = (size_t)((N + b - 1) / b);
    const size_t ck = (units * C * BD * BD * 4 + 255) & ~(size_t)255;
    return ck + units * 2 * BD * 4;
}

hipError_t launch_bwd_linear(const BwdArgs& a, hipStream_t stream)
{
    const int units = a.f.B * a.f.H;
    const size_t units_z = (size_t)units, C = (size_t)((a.f.N + a.f.b - 1) / a.f.b);
    float* ckpt = static_cast<float*>(a.f.workspace);
    float* gbpart = reinterpret_cast<float*>(static_cast<char*>(a.f.workspace) +
                                             ((units_z * C * BD * BD * 4 + 255) & ~(size_t)255));
#define TTT_BWD_LAUNCH(KIND, S)                                                                                 \
    hipLaunchKernelGGL((bwd_linear_kernel<KIND, S>), dim3(units), dim3(BT), 0, stream, a.f.H, a.f.N, a.f.b,     \
                       static_cast<const S*>(a.f.Q), static_cast<const S*>(a.f.K), static_cast<const S*>(a.f.V), \
                       a.f.eta, a.f.eta_const, a.f.W0, a.f.gamma, a.f.beta, a.f.eps, a.dZ, a.dW_end, a.dQ, a.dK, \
                       a.dV, a.deta, a.dW0, ckpt, gbpart)
    if (a.f.kind == 0 && a.f.dtype == 0) TTT_BWD_LAUNCH(0, float);
    else if (a.f.kind == 0) TTT_BWD_LAUNCH(0, uint16_t);
    else if (a.f.dtype == 0) TTT_BWD_LAUNCH(1, float);
    else TTT_BWD_LAUNCH(1, uint16_t);
#undef TTT_BWD_LAUNCH
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.f.kind == 0) return err;
    hipLaunchKernelGGL(bwd_gamma_beta_kernel, dim3(a.f.H), dim3(2 * BD), 0, stream, a.f.B, a.f.H, gbpart, a.dgamma,
                       a.dbeta);
    return hipGetLastError();
}

}  // namespace ttt
