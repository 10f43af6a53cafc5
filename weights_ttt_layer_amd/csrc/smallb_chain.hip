// smallb_chain.hip -- TTT-Linear forward (plain and LayerNorm+residual inner
// model), d = 64, 1 <= b <= 16, token streams as one bf16 term (bf16 input) or
// two (fp32 streams carried as hi + lo planes): the chunk-to-chunk chain on one
// wave, the state and the outputs on ten more.
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
// The one quantity a chunk needs from its predecessor before it can form its
// gradient is its pre-activation H_K. Substituting the state update,
//     H_K(c+1) = K_{c+1} W_{c+1} = A_{c+1} - P_{c+1} Gt_c,
//     A_{c+1} = K_{c+1} W_c,   P_{c+1} = K_{c+1} K_c^T  (16 x 16),
// and neither A_{c+1} nor P_{c+1} depends on Gt_c. The serial chain from Gt_c
// to Gt_{c+1} is therefore one 16x16 by 16x64 product and the gradient of 16
// rows; the state update, A_{c+2}, the outputs and all memory traffic run
// beside it. (The association is exact in real arithmetic; rounding differs
// from forming K_{c+1} W_{c+1} directly by the same 2^-16 order.)
//
// One workgroup of eleven waves per (sequence, head) unit. Waves are placed on
// the four SIMDs round-robin, so waves 4 and 8 share the chain's SIMD; they get
// the light roles. A state wave issues more per chunk than an output wave, so
// SIMD 3 (waves 3, 7) takes two state waves and SIMDs 1, 2 one state and two
// output waves each.
//  * wave 0, the chain: X^T = A^T + (-Gt_prev)^T P^T (v_mfma_f32_16x16x16_bf16,
//    four 16-feature tiles). Its C layout holds ONE token per lane (lane
//    (g, n): token n, features 16t + 4g + i), so a row statistic is 15 in-lane
//    adds and lane swaps (two statistics share three swaps). It writes -Gt as two bf16 terms into LDS, where
//    the transpose read hands it back as the A operand of the next chunk's
//    product. Everything it needs for a chunk except A arrives a chunk early:
//    P^T, the residual input and eta are read before it writes -Gt (their
//    latency hides behind the splits), and the -Gt read-back stays in flight
//    across the barrier, which waits only for what was issued before those
//    eight reads. It runs at raised wave priority and touches no global
//    memory.
//  * waves 1, 2, 3, 7, the state: the wave of tile b keeps W[:, 16b..16b+16)
//    in fp32 MFMA accumulators (C layout, rows = input features) and per chunk
//    computes W += K^T (-Gt) (16x16x32, the two terms of Gt stacked along k),
//    the A^T tile b of the next chunk and the Q W part of H_Q^T tile b (W^T as
//    the A operand, k in a permuted order that the B operand reads to match).
//  * waves 5, 6, 9, 10, the outputs: the wave of tile b adds the causal term
//    -Gt^T tril(S)^T to H_Q^T tile b and forms the output rows of its 16
//    features.
//  * wave 4 issues every global->LDS load of the Q/K/V/eta ring (its
//    vector-memory counter holds nothing else, so it can be waited on exactly)
//    and forms, two chunks ahead, P^T = K_c K_{c+1}^T and the causal part of
//    S^T = K_c Q_c^T (its C layout is the B operand of the causal term), both
//    as two bf16 terms; wave 8 forms the residual input of the chain's
//    gradient two chunks ahead.
// One workgroup barrier per chunk (LDS-only fence: the ring loads stay in
// flight); every exchanged tile is double-buffered by chunk parity. The output
// LayerNorm needs all 64 features of a row, so its partial sums cross the
// next barrier and a chunk's Z rows are written two chunks after its step.
//
// Precision as elsewhere: fp32 operands (state, gradient, scores, P) as two
// bf16 terms, products keeping the pairs (hi, hi), (hi, lo), (lo, hi); bf16
// token streams exact in one term, two-term streams as two planes (TIN = 2);
// fp32 accumulation.
#include "device_common.h"
#include "kernels.h"

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int NWAVE = 11;
constexpr int NTHR = 64 * NWAVE;
// Ring geometry per stream term count: slots, and chunks requested ahead of
// the one being stepped (slots of chunks c-2 .. c+2 are read during step c).
template <int TIN> struct RingGeom {
    static constexpr int SLOTS = TIN == 1 ? 12 : 8;
    static constexpr int AHEAD = TIN == 1 ? 8 : 5;
    static_assert(SLOTS >= AHEAD + 3, "slot reuse");
};

// One chunk of the ring: per stream term, [token][feature] bf16 tiles of 16
// rows x 128 bytes, 16-byte piece p of row r stored at slot p ^ (r & 7).
template <int TIN>
struct alignas(16) ChainSlot {
    uint16_t k[TIN][16 * D];
    uint16_t q[TIN][16 * D];
    uint16_t v[TIN][16 * D];
    float eta[64];           // rows 0..15 used
};

template <int TIN>
struct alignas(16) ChainSmem {
    ChainSlot<TIN> ring[RingGeom<TIN>::SLOTS];
    float4 xa[2][4][64];          // A^T of a chunk, tile t, lane order of the chain's C layout
    float4 xq[2][4][64];          // Q W part of H_Q^T of a chunk, same layout
    float4 xc[2][4][64];          // residual input of the gradient (LN: 2 gamma (K - V + beta); plain: V)
    uint2 xp[2][2][64];           // P^T of a chunk, two bf16 terms, B-operand lane order
    uint2 xst[4][2][64];          // tril(S)^T of a chunk (slot c % 4), two bf16 terms, same order
    uint16_t gt[2][2][16 * D];    // -Gt of a chunk, two bf16 terms, [token][feature] tiles
    float2 xs[2][16][4];          // output LayerNorm partial sums [token][state wave]
    float wrow[4][D];             // LN kind: partial row sums of W0 over each state wave's 16 columns
};

// Byte offset of element col (a multiple of 4) of row r in a ring/gradient tile.
__device__ __forceinline__ int toff(int r, int col)
{
    return r * 128 + (((col >> 3) ^ (r & 7)) << 4) + (col & 7) * 2;
}

// Transpose read: within each block of 16 lanes, lane j addresses row
// row0 + j/4, elements col0 + 4(j%4) .. +3, and receives column col0 + j of
// rows row0 .. row0+3. Called with row = row0 + n/4, col = col0 + 4(n%4).
__device__ __forceinline__ bf16x4 tr4(const uint16_t* tile, int row, int col)
{
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_bf16x4*)(reinterpret_cast<const char*>(tile) + toff(row, col)));
}

__device__ __forceinline__ uint2 ld8(const uint16_t* tile, int row, int col)
{
    return *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(tile) + toff(row, col));
}

__device__ __forceinline__ bf16x8 ld16(const uint16_t* tile, int row, int col)
{
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + toff(row, col));
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b)
{
    const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
    return __builtin_bit_cast(bf16x8, make_uint4(ua.x, ua.y, ub.x, ub.y));
}

__device__ __forceinline__ bf16x8 cat8(uint2 a, uint2 b)
{
    return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

__device__ __forceinline__ float4 unpack4(uint2 v)
{
    return make_float4(__builtin_bit_cast(float, v.x << 16), __builtin_bit_cast(float, v.x & 0xFFFF0000u),
                       __builtin_bit_cast(float, v.y << 16), __builtin_bit_cast(float, v.y & 0xFFFF0000u));
}

// Workgroup barrier ordering LDS only: the ring loads stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(N), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Ring loads of chunk j (rows j*b .. j*b+15, clamped to the sequence): per
// stream term, K, Q, V two 1 KB instructions each, plus one for eta when it is
// per token. Term s of a stream is the plane at element offset s * plane.
template <int TIN, bool PT>
__device__ __forceinline__ void issue_chunk(ChainSmem<TIN>& sm, int j, int lane, int N, int b, size_t plane,
                                            const uint16_t* Qu, const uint16_t* Ku, const uint16_t* Vu,
                                            const float* etau)
{
    ChainSlot<TIN>& s = sm.ring[j % RingGeom<TIN>::SLOTS];
    const int t0 = j * b;
#pragma unroll
    for (int ins = 0; ins < 2; ++ins) {
        const int sl = ins * 64 + lane;
        const int r = sl >> 3, p = (sl & 7) ^ (r & 7);
        const size_t off = (size_t)min(t0 + r, N - 1) * D + p * 8;
#pragma unroll
        for (int tm = 0; tm < TIN; ++tm) {
            dma16(Ku + tm * plane + off, __builtin_amdgcn_readfirstlane(lds_addr(s.k[tm]) + ins * 1024));
            dma16(Qu + tm * plane + off, __builtin_amdgcn_readfirstlane(lds_addr(s.q[tm]) + ins * 1024));
            dma16(Vu + tm * plane + off, __builtin_amdgcn_readfirstlane(lds_addr(s.v[tm]) + ins * 1024));
        }
    }
    if constexpr (PT) dma4(etau + min(t0 + min(lane, 15), N - 1), __builtin_amdgcn_readfirstlane(lds_addr(s.eta)));
}

// Four consecutive stream elements (row, col .. col+3) as fp32, all terms summed.
template <int TIN>
__device__ __forceinline__ float4 stream4(const uint16_t (&t)[TIN][16 * D], int row, int col)
{
    float4 v = unpack4(ld8(t[0], row, col));
    if constexpr (TIN == 2) {
        const float4 l = unpack4(ld8(t[1], row, col));
        v = make_float4(v.x + l.x, v.y + l.y, v.z + l.z, v.w + l.w);
    }
    return v;
}

// ---------------------------------------------------------------------------
// The chain wave
// ---------------------------------------------------------------------------

// What the chain reads for a chunk before that chunk's barrier: -Gt of the
// previous chunk as A operands, P^T, the residual input and eta.
struct ChainPre {
    bf16x4 ga0[4], ga1[4];
    bf16x4 pb0, pb1;
    float cp[16];
    float eta;
};

template <int TIN, bool PT>
__device__ __forceinline__ void chain_read_ops(const ChainSmem<TIN>& sm, int c, int g, int n, int lane,
                                               float eta_const, ChainPre& pre)
{
    const int par = c & 1;
    if (c > 0) {
        pre.pb0 = __builtin_bit_cast(bf16x4, sm.xp[par][0][lane]);
        pre.pb1 = __builtin_bit_cast(bf16x4, sm.xp[par][1][lane]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float4 r = sm.xc[par][t][lane];
        pre.cp[4 * t] = r.x;
        pre.cp[4 * t + 1] = r.y;
        pre.cp[4 * t + 2] = r.z;
        pre.cp[4 * t + 3] = r.w;
    }
    // rows past the sequence's end are masked where eta is used
    pre.eta = eta_const;
    if constexpr (PT) pre.eta = sm.ring[c % RingGeom<TIN>::SLOTS].eta[n];
}

// -Gt_c (written by the chain itself) as the A operands of step c + 1.
template <int TIN>
__device__ __forceinline__ void chain_read_ga(const ChainSmem<TIN>& sm, int c, int g, int n, ChainPre& pre)
{
    const uint16_t* g0 = sm.gt[c & 1][0];
    const uint16_t* g1 = sm.gt[c & 1][1];
    const int row = 4 * g + (n >> 2);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        pre.ga0[t] = tr4(g0, row, 16 * t + 4 * (n & 3));
        pre.ga1[t] = tr4(g1, row, 16 * t + 4 * (n & 3));
    }
}

// The chain's barrier with its eight -Gt reads in flight: LDS operations of one
// wave complete in order, so at most eight outstanding means everything before
// them (its -Gt writes, the other operand reads) is done. The reads only touch
// the -Gt buffer of this chunk, which no wave writes before the chain itself
// does two chunks later.
__device__ __forceinline__ void chain_barrier_ga_pending()
{
    asm volatile("s_waitcnt lgkmcnt(8)\n\ts_barrier" ::: "memory");
}

// One chain step: -Gt_c from A_c^T and the prefetched operands.
template <int KIND, int TIN, bool PT>
__device__ __forceinline__ void chain_step(ChainSmem<TIN>& sm, int c, int C, int N, int b, int g, int n, int lane,
                                           ChainPre& pre, float eta_const, const float (&g2)[16], float eps)
{
    const float eta_c = (n < min(b, N - c * b)) ? pre.eta : 0.f;
    const int par = c & 1;
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float4 a = sm.xa[par][t][lane];
        acc[t][0] = a.x;
        acc[t][1] = a.y;
        acc[t][2] = a.z;
        acc[t][3] = a.w;
    }
    __builtin_amdgcn_sched_barrier(0);   // the four reads go out together
    if (c > 0) {
        // X^T += (-Gt_{c-1})^T P_c^T : A = -Gt^T tile t (k = tokens of c-1), B = P^T
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = mfma_16x16x16(pre.ga1[t], pre.pb0, acc[t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = mfma_16x16x16(pre.ga0[t], pre.pb1, acc[t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = mfma_16x16x16(pre.ga0[t], pre.pb0, acc[t]);
    }

    float ng[16];   // -Gt of token n, features 16t + 4g + i at [4t + i]
    if constexpr (KIND == 1) {
        // LayerNorm forward statistics of the row, then its backward
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float x = acc[j >> 2][j & 3];
            s1 += x;
            s2 = fmaf(x, x, s2);
        }
        xrow4_sum2(s1, s2);
        const float mu = s1 * (1.f / D);
        const float rs = __builtin_amdgcn_rsqf(fmaxf(s2 * (1.f / D) - mu * mu, 0.f) + eps);
        const float nmr = -mu * rs;
        float xh[16], dx[16];
        float u1 = 0.f, u2 = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            xh[j] = fmaf(acc[j >> 2][j & 3], rs, nmr);
            dx[j] = fmaf(g2[j], xh[j], pre.cp[j]);   // gamma * d loss / d LN
            u1 += dx[j];
            u2 = fmaf(dx[j], xh[j], u2);
        }
        xrow4_sum2(u1, u2);
        // -eta rs (dx - mean(dx) - xh mean(dx xh))
        const float sc = -eta_c * rs;
        const float ca = -(u2 * (1.f / D)) * sc;
        const float cb = -(u1 * (1.f / D)) * sc;
#pragma unroll
        for (int j = 0; j < 16; ++j) ng[j] = fmaf(xh[j], ca, fmaf(dx[j], sc, cb));
    } else {
        // -2 eta (X - V)
        const float sc = 2.f * eta_c;
#pragma unroll
        for (int j = 0; j < 16; ++j) ng[j] = (pre.cp[j] - acc[j >> 2][j & 3]) * sc;
    }

    // the operands of chunk c + 1 (every use of this chunk's is above); their reads
    // complete behind the splits and writes below
    // (read unconditionally: past the last chunk they are in-bounds LDS reads whose
    // values go unused, and straight-line code keeps the wait counts exact)
    chain_read_ops<TIN, PT>(sm, c + 1, g, n, lane, eta_const, pre);
    asm volatile("" ::: "memory");
    char* gh = reinterpret_cast<char*>(sm.gt[par][0]);
    char* gl = reinterpret_cast<char*>(sm.gt[par][1]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t p01[2], p23[2];
        split_pair<2>(ng[4 * t], ng[4 * t + 1], p01);
        split_pair<2>(ng[4 * t + 2], ng[4 * t + 3], p23);
        const int off = toff(n, 16 * t + 4 * g);
        *reinterpret_cast<uint2*>(gh + off) = make_uint2(p01[0], p23[0]);
        *reinterpret_cast<uint2*>(gl + off) = make_uint2(p01[1], p23[1]);
    }
    // its own -Gt_c back as the next step's A operands (LDS ops of one wave are ordered)
    chain_read_ga<TIN>(sm, c, g, n, pre);
}

template <int KIND, int TIN, bool PT>
__device__ __forceinline__ void chain_role(ChainSmem<TIN>& sm, int lane, int h, int N, int b, int C,
                                           float eta_const, const float* gamma, float eps)
{
    const int g = lane >> 4, n = lane & 15;
    __builtin_amdgcn_s_setprio(3);

    float g2[16];   // 2 gamma^2 of features 16t + 4g + i
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        float gm = 0.f;
        if constexpr (KIND == 1) gm = gamma[h * D + 16 * (j >> 2) + 4 * g + (j & 3)];
        g2[j] = 2.f * gm * gm;
    }
    lds_barrier();
    lds_barrier();
    ChainPre pre;
    if (C > 0) chain_read_ops<TIN, PT>(sm, 0, g, n, lane, eta_const, pre);
    for (int c = 0; c < C + 2; ++c) {
        if (c < C) {
            chain_step<KIND, TIN, PT>(sm, c, C, N, b, g, n, lane, pre, eta_const, g2, eps);
            chain_barrier_ga_pending();
        } else {
            lds_barrier();
        }
    }
}

// ---------------------------------------------------------------------------
// The state waves
// ---------------------------------------------------------------------------

// W^T A-operand terms for the two k-steps: lane (g, n) holds W[in][16b + n] for
// in = 32p + 4g + i (tile 2p) and 32p + 16 + 4g + i (tile 2p + 1).
__device__ __forceinline__ void split_w(const f32x4 (&Wf)[4], bf16x8 (&Wt)[2][2])
{
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const float x[8] = {Wf[2 * p][0],     Wf[2 * p][1],     Wf[2 * p][2],     Wf[2 * p][3],
                            Wf[2 * p + 1][0], Wf[2 * p + 1][1], Wf[2 * p + 1][2], Wf[2 * p + 1][3]};
        terms8<2>(x, Wt[p]);
    }
}

// W^T X^T for the 16 rows of a ring tile (X = K or Q, TIN terms): C layout
// lane (g, n) = row n, output features 16b + 4g + i. B operand in the k order
// of split_w.
template <int TIN>
__device__ __forceinline__ f32x4 wt_rows(const bf16x8 (&Wt)[2][2], const uint16_t (&xt)[TIN][16 * D], int g, int n)
{
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const bf16x8 x0 = cat8(ld8(xt[0], n, 32 * p + 4 * g), ld8(xt[0], n, 32 * p + 16 + 4 * g));
        a = mfma_16x16x32(Wt[p][1], x0, a);
        if constexpr (TIN == 2) {
            const bf16x8 x1 = cat8(ld8(xt[1], n, 32 * p + 4 * g), ld8(xt[1], n, 32 * p + 16 + 4 * g));
            a = mfma_16x16x32(Wt[p][0], x1, a);
        }
        a = mfma_16x16x32(Wt[p][0], x0, a);
    }
    return a;
}

// Row products X Y^T of two ring tiles (k = features, natural order; TIN terms
// each, pairs (hi, hi), (hi, lo), (lo, hi)): C layout lane (g, n) = X[4g + i] . Y[n].
template <int TIN>
__device__ __forceinline__ f32x4 row_dots(const uint16_t (&xt)[TIN][16 * D], const uint16_t (&yt)[TIN][16 * D], int g,
                                          int n)
{
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const bf16x8 x0 = ld16(xt[0], n, 32 * p + 8 * g), y0 = ld16(yt[0], n, 32 * p + 8 * g);
        if constexpr (TIN == 2) {
            a = mfma_16x16x32(ld16(xt[1], n, 32 * p + 8 * g), y0, a);
            a = mfma_16x16x32(x0, ld16(yt[1], n, 32 * p + 8 * g), a);
        }
        a = mfma_16x16x32(x0, y0, a);
    }
    return a;
}

template <int KIND, int TIN>
__device__ __forceinline__ void w_role(ChainSmem<TIN>& sm, int bt, int lane, int C, const float* W0u, float* Wu)
{
    constexpr int SL = RingGeom<TIN>::SLOTS;
    const int g = lane >> 4, n = lane & 15;
    __builtin_amdgcn_s_setprio(2);

    // resident state: Wf[a][i] = W[16a + 4g + i][16b + n]
    f32x4 Wf[4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) Wf[a][i] = W0u[(16 * a + 4 * g + i) * D + 16 * bt + n];
    // LN kind: the state is carried with each row's mean over the output
    // features removed. LayerNorm ignores a constant added to a whole row, so
    // K W' and K W have the same LayerNorm and gradient; and the LayerNorm
    // gradient of every token sums to zero over the features, so the update
    // K^T Gt never changes the row means. The removed means are added back to
    // W_end. With it, pre-activation rows have a near-zero mean whatever W0
    // holds, so the one-pass variance and the two-term operands keep their
    // relative precision.
    float wmean[4][4] = {};
    if constexpr (KIND == 1) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s = row16_sum(Wf[a][i]);
                if (n == 0) sm.wrow[bt][16 * a + 4 * g + i] = s;
            }
    }

    lds_barrier();                       // chunks 0 and 1 in LDS
    if constexpr (KIND == 1) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * a + 4 * g + i;
                wmean[a][i] = ((sm.wrow[0][r] + sm.wrow[1][r]) + (sm.wrow[2][r] + sm.wrow[3][r])) * (1.f / D);
                Wf[a][i] -= wmean[a][i];
            }
    }
    bf16x8 Wt[2][2];
    split_w(Wf, Wt);
    if (C > 0) {
        const f32x4 a = wt_rows<TIN>(Wt, sm.ring[0].k, g, n);
        sm.xa[0][bt][lane] = make_float4(a[0], a[1], a[2], a[3]);
    }
    lds_barrier();

    for (int c = 0; c < C + 2; ++c) {
        if (c >= 1 && c <= C) {
            // W_c = W_{c-1} + K_{c-1}^T (-Gt_{c-1}); k = 16 tokens x 2 terms of Gt stacked
            const auto& kt = sm.ring[(c - 1) % SL].k;
            const uint16_t* gtt = sm.gt[(c - 1) & 1][g >> 1];
            const int row = 8 * (g & 1) + (n >> 2);
            const int cq = 4 * (n & 3);
            const bf16x8 gb = cat8(tr4(gtt, row, 16 * bt + cq), tr4(gtt, row + 4, 16 * bt + cq));
            bf16x4 gh = {};
            if constexpr (TIN == 2) gh = tr4(sm.gt[(c - 1) & 1][0], 4 * g + (n >> 2), 16 * bt + cq);
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const bf16x8 ka = cat8(tr4(kt[0], row, 16 * a + cq), tr4(kt[0], row + 4, 16 * a + cq));
                Wf[a] = mfma_16x16x32(ka, gb, Wf[a]);
                if constexpr (TIN == 2)   // the lo term of K against the hi term of Gt
                    Wf[a] = mfma_16x16x16(tr4(kt[1], 4 * g + (n >> 2), 16 * a + cq), gh, Wf[a]);
            }
            if (c < C) split_w(Wf, Wt);
        }
        if (c + 1 < C) {
            const f32x4 a = wt_rows<TIN>(Wt, sm.ring[(c + 1) % SL].k, g, n);
            sm.xa[(c + 1) & 1][bt][lane] = make_float4(a[0], a[1], a[2], a[3]);
        }
        if (c < C) {
            const f32x4 q = wt_rows<TIN>(Wt, sm.ring[c % SL].q, g, n);
            sm.xq[c & 1][bt][lane] = make_float4(q[0], q[1], q[2], q[3]);
        }
        lds_barrier();
    }

    // W_end = W0 + (accumulated change): W0 - mean is formed again with the
    // rounding it had at the start, so a state that never moved comes back bit
    // for bit. (W_end may be W0: every entry is read and written by one lane.)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const size_t o = (size_t)(16 * a + 4 * g + i) * D + 16 * bt + n;
            float v = Wf[a][i];
            if constexpr (KIND == 1) {
                const float w0 = W0u[o];
                v = w0 + (v - (w0 - wmean[a][i]));
            }
            Wu[o] = v;
        }
}

// ---------------------------------------------------------------------------
// The loader (and P^T) wave and the residual-input wave
// ---------------------------------------------------------------------------

// P_j^T = K_{j-1} K_j^T as two bf16 terms, for the chain's chunk j.
template <int TIN>
__device__ __forceinline__ void publish_p(ChainSmem<TIN>& sm, int j, int g, int n, int lane)
{
    constexpr int SL = RingGeom<TIN>::SLOTS;
    const f32x4 p = row_dots<TIN>(sm.ring[(j - 1) % SL].k, sm.ring[j % SL].k, g, n);
    const float x[4] = {p[0], p[1], p[2], p[3]};
    bf16x4 pt[2];
    terms4<2>(x, pt);
    sm.xp[j & 1][0][lane] = __builtin_bit_cast(uint2, pt[0]);
    sm.xp[j & 1][1][lane] = __builtin_bit_cast(uint2, pt[1]);
}

// tril(S_j)^T = (K_j Q_j^T) with key 4g + i <= query n, as two bf16 terms, for
// the output waves' causal term of chunk j.
template <int TIN>
__device__ __forceinline__ void publish_s(ChainSmem<TIN>& sm, int j, int g, int n, int lane)
{
    const ChainSlot<TIN>& s = sm.ring[j % RingGeom<TIN>::SLOTS];
    const f32x4 st = row_dots<TIN>(s.k, s.q, g, n);
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (4 * g + i <= n) ? st[i] : 0.f;
    bf16x4 sb[2];
    terms4<2>(x, sb);
    sm.xst[j & 3][0][lane] = __builtin_bit_cast(uint2, sb[0]);
    sm.xst[j & 3][1][lane] = __builtin_bit_cast(uint2, sb[1]);
}

template <int TIN, bool PT>
__device__ __forceinline__ void loader_role(ChainSmem<TIN>& sm, int lane, int N, int b, int C, size_t plane,
                                            const uint16_t* Qu, const uint16_t* Ku, const uint16_t* Vu,
                                            const float* etau)
{
    constexpr int DPC = 6 * TIN + (PT ? 1 : 0);   // ring-load instructions per chunk
    constexpr int AH = RingGeom<TIN>::AHEAD;
    const int g = lane >> 4, n = lane & 15;
    const int npro = min(AH, C);
    for (int j = 0; j < npro; ++j) issue_chunk<TIN, PT>(sm, j, lane, N, b, plane, Qu, Ku, Vu, etau);
    if (C >= AH) wait_vm<DPC * (AH - 2)>(); else wait_vm<0>();   // chunks 0, 1
    lds_barrier();
    if (C > 1) publish_p<TIN>(sm, 1, g, n, lane);
    if (C > 0) publish_s<TIN>(sm, 0, g, n, lane);
    if (C > 1) publish_s<TIN>(sm, 1, g, n, lane);
    if (C >= AH) wait_vm<DPC * (AH - 3)>(); else wait_vm<0>();   // chunk 2
    lds_barrier();
    for (int c = 0; c < C + 2; ++c) {
        if (c + AH < C) issue_chunk<TIN, PT>(sm, c + AH, lane, N, b, plane, Qu, Ku, Vu, etau);
        if (c + 2 < C) {
            publish_p<TIN>(sm, c + 2, g, n, lane);
            publish_s<TIN>(sm, c + 2, g, n, lane);   // slot (c+2) % 4 was last read at step c-2
        }
        // chunk c + 3 is read after this barrier
        if (c + AH < C) wait_vm<DPC * (AH - 3)>(); else wait_vm<0>();
        lds_barrier();
    }
}

// Residual input of the chain's gradient for chunk j, all four tiles, in the
// chain's lane order (LN: 2 gamma (K - V + beta); plain: V).
template <int KIND, int TIN>
__device__ __forceinline__ void publish_c(ChainSmem<TIN>& sm, int j, int g, int n, int lane, const float (&c2g)[16],
                                          const float (&c2gb)[16])
{
    const ChainSlot<TIN>& s = sm.ring[j % RingGeom<TIN>::SLOTS];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int f = 16 * t + 4 * g;
        const float4 vv = stream4<TIN>(s.v, n, f);
        float4 r = vv;
        if constexpr (KIND == 1) {
            const float4 kk = stream4<TIN>(s.k, n, f);
            r = make_float4(fmaf(kk.x - vv.x, c2g[4 * t], c2gb[4 * t]), fmaf(kk.y - vv.y, c2g[4 * t + 1], c2gb[4 * t + 1]),
                            fmaf(kk.z - vv.z, c2g[4 * t + 2], c2gb[4 * t + 2]),
                            fmaf(kk.w - vv.w, c2g[4 * t + 3], c2gb[4 * t + 3]));
        }
        sm.xc[j & 1][t][lane] = r;
    }
}

template <int KIND, int TIN>
__device__ __forceinline__ void resid_role(ChainSmem<TIN>& sm, int lane, int h, int C, const float* gamma,
                                           const float* beta)
{
    const int g = lane >> 4, n = lane & 15;
    float c2g[16], c2gb[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int f = 16 * (j >> 2) + 4 * g + (j & 3);
        const float gm = (KIND == 1) ? gamma[h * D + f] : 0.f;
        const float bt = (KIND == 1) ? beta[h * D + f] : 0.f;
        c2g[j] = 2.f * gm;
        c2gb[j] = 2.f * gm * bt;
    }
    lds_barrier();
    if (C > 0) publish_c<KIND, TIN>(sm, 0, g, n, lane, c2g, c2gb);
    if (C > 1) publish_c<KIND, TIN>(sm, 1, g, n, lane, c2g, c2gb);
    lds_barrier();
    for (int c = 0; c < C + 2; ++c) {
        if (c + 2 < C) publish_c<KIND, TIN>(sm, c + 2, g, n, lane, c2g, c2gb);
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// The output waves
// ---------------------------------------------------------------------------

template <int KIND, int TIN>
__device__ __forceinline__ void out_role(ChainSmem<TIN>& sm, int bt, int lane, int h, int N, int b, int C,
                                         const float* gamma, const float* beta, float eps, float* Zu)
{
    constexpr int SL = RingGeom<TIN>::SLOTS;
    const int g = lane >> 4, n = lane & 15;
    const int fo = 16 * bt + 4 * g;   // first of this lane's four output features
    float gam[4], bet[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        gam[i] = (KIND == 1) ? gamma[h * D + fo + i] : 0.f;
        bet[i] = (KIND == 1) ? beta[h * D + fo + i] : 0.f;
    }
    lds_barrier();
    lds_barrier();

    f32x4 xq2 = {0.f, 0.f, 0.f, 0.f};   // final H_Q^T tile b of chunk c-2
    bf16x4 sb1[2] = {};                  // tril(S_{c-1})^T terms

    for (int c = 0; c < C + 2; ++c) {
        const int par = c & 1;
        f32x4 xq1 = {0.f, 0.f, 0.f, 0.f};
        if (c >= 1 && c <= C) {
            // H_Q^T(c-1) = Q W part + (-Gt_{c-1})^T tril(S_{c-1})^T
            const float4 q = sm.xq[par ^ 1][bt][lane];
            xq1[0] = q.x;
            xq1[1] = q.y;
            xq1[2] = q.z;
            xq1[3] = q.w;
            const int row = 4 * g + (n >> 2);
            const int col = 16 * bt + 4 * (n & 3);
            const bf16x4 ga0 = tr4(sm.gt[par ^ 1][0], row, col);
            const bf16x4 ga1 = tr4(sm.gt[par ^ 1][1], row, col);
            xq1 = mfma_16x16x16(ga1, sb1[0], xq1);
            xq1 = mfma_16x16x16(ga0, sb1[1], xq1);
            xq1 = mfma_16x16x16(ga0, sb1[0], xq1);
        }
        bf16x4 sbn[2] = {};
        if (c < C) {
            // tril(S_c)^T terms, formed by the loader wave two chunks ahead
            sbn[0] = __builtin_bit_cast(bf16x4, sm.xst[c & 3][0][lane]);
            sbn[1] = __builtin_bit_cast(bf16x4, sm.xst[c & 3][1][lane]);
        }
        if (c >= 1 && c <= C) {
            const int m = c - 1;
            if constexpr (KIND == 1) {
                // partial output-LayerNorm sums of chunk c-1 over this wave's 16 features
                float s1 = (xq1[0] + xq1[1]) + (xq1[2] + xq1[3]);
                float s2 = (xq1[0] * xq1[0] + xq1[1] * xq1[1]) + (xq1[2] * xq1[2] + xq1[3] * xq1[3]);
                xrow4_sum2(s1, s2);
                if (g == 0) sm.xs[par][n][bt] = make_float2(s1, s2);
            } else {
                if (n < min(b, N - m * b))
                    *reinterpret_cast<float4*>(Zu + (size_t)(m * b + n) * D + fo) =
                        make_float4(xq1[0], xq1[1], xq1[2], xq1[3]);
            }
        }
        if constexpr (KIND == 1) {
            if (c >= 2) {
                // Z rows of chunk c-2: Q + gamma LN(H_Q) + beta
                const int m = c - 2;
                const float4 pa = *reinterpret_cast<const float4*>(&sm.xs[par ^ 1][n][0]);
                const float4 pb = *reinterpret_cast<const float4*>(&sm.xs[par ^ 1][n][2]);
                const float S1 = (pa.x + pa.z) + (pb.x + pb.z);
                const float S2 = (pa.y + pa.w) + (pb.y + pb.w);
                const float mu = S1 * (1.f / D);
                const float rs = __builtin_amdgcn_rsqf(fmaxf(S2 * (1.f / D) - mu * mu, 0.f) + eps);
                const float4 q = stream4<TIN>(sm.ring[m % SL].q, n, fo);
                const float qv[4] = {q.x, q.y, q.z, q.w};
                float z[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) z[i] = qv[i] + gam[i] * ((xq2[i] - mu) * rs) + bet[i];
                if (n < min(b, N - m * b))
                    *reinterpret_cast<float4*>(Zu + (size_t)(m * b + n) * D + fo) = make_float4(z[0], z[1], z[2], z[3]);
            }
        }
        xq2 = xq1;
        sb1[0] = sbn[0];
        sb1[1] = sbn[1];
        lds_barrier();
    }
}

template <int KIND, int TIN, bool PT>
__global__ void __launch_bounds__(NTHR)
smallb_chain_kernel(int H, int N, int b, size_t plane, const uint16_t* __restrict__ Qg,
                    const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
                    const float* __restrict__ etag, float eta_const, const float* __restrict__ W0,
                    const float* __restrict__ gamma, const float* __restrict__ beta, float eps,
                    float* __restrict__ Zg, float* __restrict__ Wend)
{
    __shared__ ChainSmem<TIN> sm;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const size_t unit = blockIdx.x;
    const int h = (int)(unit % H);
    const int C = (N + b - 1) / b;
    // roles by wave index (wave w runs on SIMD w % 4; 4 and 8 share the chain's)
    if (w == 0) {
        chain_role<KIND, TIN, PT>(sm, lane, h, N, b, C, eta_const, gamma, eps);
    } else if (w == 4) {
        loader_role<TIN, PT>(sm, lane, N, b, C, plane, Qg + unit * (size_t)N * D, Kg + unit * (size_t)N * D,
                             Vg + unit * (size_t)N * D, PT ? etag + unit * (size_t)N : nullptr);
    } else if (w == 8) {
        resid_role<KIND, TIN>(sm, lane, h, C, gamma, beta);
    } else if (w <= 3 || w == 7) {
        const int bt = (w == 7) ? 3 : w - 1;
        w_role<KIND, TIN>(sm, bt, lane, C, W0 + unit * (size_t)D * D, Wend + unit * (size_t)D * D);
    } else {
        const int bt = (w <= 6) ? w - 5 : w - 7;
        out_role<KIND, TIN>(sm, bt, lane, h, N, b, C, gamma, beta, eps, Zg + unit * (size_t)N * D);
    }
}

template <int KIND, int TIN, bool PT>
hipError_t launch_typed(const LinearArgs& a, hipStream_t stream)
{
    const size_t plane = (size_t)a.B * a.H * a.N * D;
    hipLaunchKernelGGL((smallb_chain_kernel<KIND, TIN, PT>), dim3(a.B * a.H), dim3(NTHR), 0, stream, a.H, a.N, a.b,
                       plane, static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                       static_cast<const uint16_t*>(a.V), a.eta, a.eta_const, a.W0, a.gamma, a.beta, a.eps,
                       a.Z, a.W_end);
    return hipGetLastError();
}

template <int TIN>
hipError_t launch_terms(const LinearArgs& a, hipStream_t stream)
{
    if (a.kind == 1) return a.eta ? launch_typed<1, TIN, true>(a, stream) : launch_typed<1, TIN, false>(a, stream);
    return a.eta ? launch_typed<0, TIN, true>(a, stream) : launch_typed<0, TIN, false>(a, stream);
}

}  // namespace

hipError_t launch_smallb_chain(const LinearArgs& a, hipStream_t stream) { return launch_terms<1>(a, stream); }

hipError_t launch_smallb_chain_terms2(const LinearArgs& a, hipStream_t stream) { return launch_terms<2>(a, stream); }

}  // namespace ttt
