// large_chunk.hip -- TTT-Linear forward, plain f(x) = x W, for large mini-batches
// (b >= 256, b % 128 == 0, d = 128, N % 128 == 0), bf16 token streams.
//
// Large chunks are what the page "Test-Time Training Done Right" (abstract)
// proposes against the low utilisation of small mini-batches; the computation
// is the same mini-batch dual form (page "Test-Time Training: Linear Complexity
// Beyond Attention", section "4. Mini-Batch Parallelism (Dual Formulation)"):
//     E_c = K_c W_c - V_c,   W_{c+1} = W_c - 2 K_c^T diag(eta) E_c,
//     Z_c = Q_c W_c - 2 tril(Q_c K_c^T) diag(eta) E_c.
// For plain f the chunk update is affine in W:
//     W_{c+1} = W_c - M_c W_c + B_c,   M_c = K_c^T D K_c,  B_c = K_c^T D V_c,
// D = diag(2 eta). The path runs three kernels on one stream:
//   lc_gram  : M_c and B_c for every (unit, chunk) at once (no dependence on W);
//   lc_scan  : the recurrence W_c -> W_{c+1} (one workgroup per (unit,
//              32-column block)); writes every W_c^T as two bf16 terms and W_end;
//   lc_chunk : Z of every (unit, chunk) at once from W_c, fused: the chunk's
//              residuals, the causal term and the output in one pass over
//              Q, K, V (sub-blocks of 64 tokens, see below);
//   lc_apply : instead of lc_chunk for block-causal outputs, Z_c = Q_c W_c or
//              Q_c W_{c+1} (no causal term inside a chunk).
// Workspace (caller-provided): M, B (fp32), W_c^T terms (bf16).
//
// Precision: every product involving an fp32 quantity (state, gradient, the
// causal scores q.k) uses two bf16 terms (16 significant bits); bf16 token
// streams are exact in one term. All accumulation is fp32.
//
// MFMA v_mfma_f32_32x32x16_bf16 throughout. Token-major operands (the token
// index contracted in K^T K, K^T V, K^T Gn) are read from row-major LDS tiles
// with the gfx950 transpose read ds_read_b64_tr_b16.
#include "device_common.h"
#include "kernels.h"

namespace ttt {
namespace {

constexpr int LD = 128;          // head dim of this path
constexpr int LT = 256;          // threads per workgroup
constexpr int TB = 128;          // chunk lengths are multiples of this

// Row of a 32x32 C-layout tile held by lane half h = lane / 32 at slot i.
__device__ __forceinline__ int crow(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

struct LcLayout {
    size_t m_off, b_off, wt_off, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline LcLayout lc_layout(int units, int N, int b)
{
    const size_t C = (size_t)((N + b - 1) / b);
    LcLayout L;
    L.m_off = 0;
    L.b_off = align256(L.m_off + (size_t)units * C * LD * LD * 4);
    L.wt_off = align256(L.b_off + (size_t)units * C * LD * LD * 4);
    L.total = align256(L.wt_off + (size_t)units * (C + 1) * 2 * LD * LD * 2);
    return L;
}

typedef __attribute__((address_space(3))) void lds_void;

// LDS tiles have 256-byte rows = 16 pieces of 16 bytes; piece p of row r is
// stored at slot p ^ rsw(r). rsw is a bijection of r % 16 whose low three bits
// differ across 8 consecutive rows and whose bits 1-2 differ across 4 aligned
// rows, which keeps the row reads (8 or 16 rows, one piece) and the transpose
// reads (4 rows, two adjacent pieces) free of bank conflicts.
__device__ __forceinline__ int rsw(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }
// byte offset of piece p of row r
__device__ __forceinline__ int swz(int r, int p) { return r * 256 + ((p ^ rsw(r)) << 4); }


// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
enum : int { SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM_R = 0x020, SG_DS_R = 0x100 };
#define SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// ===========================================================================
// lc_gram: M_c = K^T D K and B_c = K^T D V for one (unit, chunk) per workgroup.
// Wave w computes row tile w of both (rows 32w..32w+31, all four column tiles),
// so one A operand (the D-scaled K^T fragment) feeds eight products. K and V
// stream through LDS in 64-token stages, GR_NST stages in flight.
//
// Outputs are written in the register order in which lc_scan consumes them:
//  * M_c, as two bf16 terms, tile (r, cc) lane by lane: lc_scan's wave w needs
//    M_c[32w + l32][k] for k = 32r + crow(8s + j, h) (its k order), which by
//    symmetry is M_c[32r + crow(8s+j, h)][32w + l32], i.e. slot 8s + j of lane
//    (l32, h) of tile (r, cc = w).  Layout [tile][term][s][lane][8].
//  * B_c, fp32, tile (r, cc) lane by lane in its C layout: [tile][q][lane][4]
//    (slots 4q .. 4q+3).
// ===========================================================================
constexpr int GR_TOK = 64;              // tokens per LDS stage
constexpr int GR_NST = 4;               // LDS stages (three in flight while one is read)

struct GramSmem {
    uint16_t k[GR_NST][GR_TOK * LD];    // [token][feature], swizzled pieces
    uint16_t v[GR_NST][GR_TOK * LD];
};

// Token-major operand fragment of a [tokens x 128] bf16 LDS tile: lane l gets
// the 8 tokens t0 + 8*(l/32) + 0..7 of feature 32*f + l%32 (two transpose reads).
__device__ __forceinline__ bf16x8 tok_major_frag(const uint16_t* tile, int t0, int f, int lane)
{
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const int q = lane >> 4, r = lane & 15;
    const int row = t0 + 8 * (q >> 1) + (r >> 2);
    const int colm = 32 * f + 16 * (q & 1) + 4 * (r & 3);
    const char* base = reinterpret_cast<const char*>(tile);
    const char* p0 = base + swz(row, colm >> 3) + (colm & 7) * 2;
    const char* p1 = base + swz(row + 4, colm >> 3) + (colm & 7) * 2;
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(p0));
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(p1));
    const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
    return __builtin_bit_cast(bf16x8, make_uint4(ua.x, ua.y, ub.x, ub.y));
}

// Fill the K and V tiles of stage s with direct LDS loads: each tile is 16
// wave instructions of 1 KB; wave w issues instructions 4w .. 4w+3 of each.
__device__ __forceinline__ void gram_dma(GramSmem& sm, int buf, int s, int w, int lane, const uint16_t* Ku,
                                         const uint16_t* Vu)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int sl = (4 * w + k) * 64 + lane;
        const int r = sl >> 4, p = (sl & 15) ^ rsw(r);
        const size_t off = (size_t)(s * GR_TOK + r) * LD + p * 8;
        dma16(Ku + off, __builtin_amdgcn_readfirstlane(lds_addr(reinterpret_cast<char*>(sm.k[buf]) + (4 * w + k) * 1024)));
        dma16(Vu + off, __builtin_amdgcn_readfirstlane(lds_addr(reinterpret_cast<char*>(sm.v[buf]) + (4 * w + k) * 1024)));
    }
}

// A operand of K^T D: the fragment itself (constant eta, D applied after the
// sum) or, with per-token eta, each token's entry times 2 eta_t as TA terms.
template <bool PER_TOKEN, int TA>
__device__ __forceinline__ void scaled_frag(const bf16x8& f, const float* eta8, bf16x8 (&out)[TA])
{
    if constexpr (PER_TOKEN) {
        const float4 e0 = *reinterpret_cast<const float4*>(eta8);
        const float4 e1 = *reinterpret_cast<const float4*>(eta8 + 4);
        const float e[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = 2.f * e[j] * (float)f[j];
        terms8<TA>(x, out);
    } else {
        out[0] = f;
    }
}

// s_waitcnt immediate: at most `vm` vector-memory operations outstanding
// (lgkmcnt and expcnt not waited for).
constexpr int vmcnt_imm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8); }

template <bool PER_TOKEN>
__global__ void __launch_bounds__(LT)
lc_gram_kernel(int N, int b, const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
               const float* __restrict__ etag, float eta_const, uint16_t* __restrict__ Mout,
               float* __restrict__ Bout)
{
    constexpr int TA = PER_TOKEN ? 2 : 1;    // terms of the D-scaled operand
    constexpr int OPS = 8;                   // direct loads per wave per stage
    __shared__ GramSmem sm;
    const int C = (N + b - 1) / b;
    const int unit = blockIdx.x / C, c = blockIdx.x % C;
    const int c0 = c * b, nt = min(b, N - c0);
    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint16_t* Ku = Kg + ((size_t)unit * N + c0) * LD;
    const uint16_t* Vu = Vg + ((size_t)unit * N + c0) * LD;
    const float* etau = PER_TOKEN ? etag + (size_t)unit * N + c0 : nullptr;

    f32x16 accB[4], accM[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        accB[t] = f32x16{};
        accM[t] = f32x16{};
    }

    // The sums are order-free, so the stages run from the end of the chunk to its
    // start (stage s holds tokens of block nstage - 1 - s): the chunk's first
    // tokens are then the most recently read when lc_chunk, which must walk the
    // chunk from its start, reads them again, and the memory-side cache can serve them.
    const int nstage = nt / GR_TOK;
#pragma unroll
    for (int s = 0; s < GR_NST - 1; ++s)
        if (s < nstage) gram_dma(sm, s, nstage - 1 - s, w, lane, Ku, Vu);
    for (int s = 0; s < nstage; ++s) {
        // stage s is this wave's oldest outstanding group of loads
        const int later = min(GR_NST - 2, nstage - 1 - s);
        if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * OPS));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(OPS));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();                                 // stage s landed everywhere; stage s-1 consumed
        if (s + GR_NST - 1 < nstage)
            gram_dma(sm, (s + GR_NST - 1) % GR_NST, nstage - s - GR_NST, w, lane, Ku, Vu);
        const uint16_t* kt = sm.k[s % GR_NST];
        const uint16_t* vt = sm.v[s % GR_NST];
        // operands of k-step ks + 1 are read while the products of ks run
        struct Ops { bf16x8 aw[TA], bv[4], bk[4]; };
        auto ops = [&](int ks, Ops& o) {
            const float* er = PER_TOKEN ? etau + (nstage - 1 - s) * GR_TOK + 16 * ks + 8 * h : nullptr;
            scaled_frag<PER_TOKEN, TA>(tok_major_frag(kt, 16 * ks, w, lane), er, o.aw);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                o.bv[t] = tok_major_frag(vt, 16 * ks, t, lane);
                o.bk[t] = tok_major_frag(kt, 16 * ks, t, lane);
            }
        };
        Ops cur;
        ops(0, cur);
#pragma unroll
        for (int ks = 0; ks < GR_TOK / 16; ++ks) {
            Ops nxt;
            if (ks + 1 < GR_TOK / 16) ops(ks + 1, nxt);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int s2 = TA - 1; s2 >= 0; --s2) {
                    accB[t] = mfma_32x32x16(cur.aw[s2], cur.bv[t], accB[t]);
                    accM[t] = mfma_32x32x16(cur.aw[s2], cur.bk[t], accM[t]);
                }
            if (ks + 1 < GR_TOK / 16) cur = nxt;
        }
        if constexpr (!PER_TOKEN) {
            SCHED_GROUP(SG_DS_R, 18);
#pragma unroll
            for (int ks = 0; ks < GR_TOK / 16; ++ks) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    if (ks + 1 < GR_TOK / 16) {
                        if (k < 2) SCHED_GROUP(SG_DS_R, 3);
                        else SCHED_GROUP(SG_DS_R, 2);
                    }
                    SCHED_GROUP(SG_MFMA, 1);
                }
            }
        }
    }

    const float scale = PER_TOKEN ? 1.f : 2.f * eta_const;
    const size_t base = ((size_t)unit * C + c) * LD * LD;
    uint16_t* Mo = Mout + 2 * base;                      // two bf16 terms per element
    float* Bo = Bout + base;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int tile = 4 * w + t;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(Bo + ((size_t)(tile * 4 + q) * 64 + lane) * 4) =
                make_float4(scale * accB[t][4 * q], scale * accB[t][4 * q + 1], scale * accB[t][4 * q + 2],
                            scale * accB[t][4 * q + 3]);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = scale * accM[t][8 * s2 + j];
            bf16x8 mt[2];
            terms8<2>(x, mt);
#pragma unroll
            for (int term = 0; term < 2; ++term)
                *reinterpret_cast<bf16x8*>(Mo + ((size_t)((tile * 2 + term) * 2 + s2) * 64 + lane) * 8) = mt[term];
        }
    }
}

// ===========================================================================
// lc_scan: W_{c+1} = W_c - M_c W_c + B_c for one (unit, 32-column block).
// Wave w holds rows [32w, 32w+32) of the block as one 32x32 C tile (acc).
// The product M_c W_c runs over k in the order 32r + crow(8s + j, h): in that
// order the B operand (rows of W_c) of k-step (r, s) is exactly what wave r
// holds in slots 8s .. 8s+7 of the same lane, so every wave publishes its
// tile's two bf16 terms lane by lane in LDS and reads the others' at its own
// lane index; the A operand comes ready-split from lc_gram in that order.
// The operands of step c+2 are requested as step c finishes. W_0 .. W_C are all
// published (W_C, the final state, for outputs taken after the last step).
// ===========================================================================
struct ScanOps {
    bf16x8 a[4][2][2];                  // M_c A operand [r][s][term]
    float4 bq[4];                       // B_c entries of this lane's C tile
};

__device__ __forceinline__ void scan_load(const uint16_t* Mg, const float* Bg, int unit, int C, int c, int w,
                                          int cb, int lane, ScanOps& o)
{
    const size_t base = ((size_t)unit * C + c) * LD * LD;
    const uint16_t* Mc = Mg + 2 * base;
    const float* Bc = Bg + base;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int term = 0; term < 2; ++term)
                o.a[r][s][term] = *reinterpret_cast<const bf16x8*>(
                    Mc + ((size_t)(((4 * r + w) * 2 + term) * 2 + s) * 64 + lane) * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o.bq[q] = *reinterpret_cast<const float4*>(Bc + ((size_t)((4 * w + cb) * 4 + q) * 64 + lane) * 4);
}

// Two bf16 terms of this lane's 16 state entries: into `pub` (lane by lane, if
// given) and into W^T of the workspace (wt: [term][column][row]).
__device__ __forceinline__ void publish_state(const f32x16& acc, uint16_t* wt, bf16x8 (*pub)[2][64], int w,
                                              int lane, int h, int colg)
{
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = acc[8 * s + j];
        bf16x8 tw[2];
        terms8<2>(x, tw);
        if (pub) {
            pub[0][s][lane] = tw[0];
            pub[1][s][lane] = tw[1];
        }
        // slots 8s .. 8s+3 and 8s+4 .. 8s+7 are rows row0 .. row0+3 and row0+8 .. row0+11
        const int row0 = 32 * w + 16 * s + 4 * h;
#pragma unroll
        for (int term = 0; term < 2; ++term) {
            const uint4 u = __builtin_bit_cast(uint4, tw[term]);
            *reinterpret_cast<uint2*>(wt + (size_t)term * LD * LD + (size_t)colg * LD + row0) = make_uint2(u.x, u.y);
            *reinterpret_cast<uint2*>(wt + (size_t)term * LD * LD + (size_t)colg * LD + row0 + 8) =
                make_uint2(u.z, u.w);
        }
    }
}

__global__ void __launch_bounds__(LT)
lc_scan_kernel(int N, int b, const float* __restrict__ W0, const uint16_t* __restrict__ Mg,
               const float* __restrict__ Bg, uint16_t* __restrict__ WT, float* __restrict__ Wend)
{
    // [buffer][wave][term][s][lane] bf16x8: W_c rows of every wave, lane by lane
    __shared__ __attribute__((aligned(16))) bf16x8 wpub[2][4][2][2][64];
    const int C = (N + b - 1) / b;
    // the four column blocks of a unit read the same M_c every step: keep them on
    // one XCD so three of the four reads hit its L2
    const int lb = xcd_tile(blockIdx.x, gridDim.x);
    const int unit = lb >> 2, cb = lb & 3;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int colg = 32 * cb + l32;   // global column of this lane

    f32x16 acc;
    const float* W0u = W0 + (size_t)unit * LD * LD;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = W0u[(32 * w + crow(i, h)) * LD + colg];

    // One step: publish W_c, then W_{c+1} = W_c - M_c W_c + B_c with the
    // operands in `o`; afterwards `o` is refilled with step c + 2's operands.
    // The two operand sets alternate by name (the loop is unrolled by two), so
    // no register copy makes the compiler wait for a refill before its use.
    auto step = [&](int c, ScanOps& o) {
        const int buf = c & 1;
        // publish W_c: two bf16 terms, lane by lane in LDS and as W_c^T in the workspace
        publish_state(acc, WT + ((size_t)unit * (C + 1) + c) * 2 * LD * LD, wpub[buf][w], w, lane, h, colg);
        __syncthreads();                                 // one barrier per step: wpub is double-buffered
        // t = M_c W_c - B_c: B_c enters as the accumulator's start, so its registers
        // are free for the refill as soon as the first product has read them
        f32x16 t;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            t[4 * q] = -o.bq[q].x;
            t[4 * q + 1] = -o.bq[q].y;
            t[4 * q + 2] = -o.bq[q].z;
            t[4 * q + 3] = -o.bq[q].w;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const bf16x8 b0 = wpub[buf][r][0][s][lane];
                const bf16x8 b1 = wpub[buf][r][1][s][lane];
                t = mfma_32x32x16(o.a[r][s][1], b0, t);
                t = mfma_32x32x16(o.a[r][s][0], b1, t);
                t = mfma_32x32x16(o.a[r][s][0], b0, t);
            }
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] -= t[i];
        if (c + 2 < C) scan_load(Mg, Bg, unit, C, c + 2, w, cb, lane, o);
    };

    ScanOps oA, oB;
    scan_load(Mg, Bg, unit, C, 0, w, cb, lane, oA);
    if (C > 1) scan_load(Mg, Bg, unit, C, 1, w, cb, lane, oB);
    for (int c = 0; c < C; c += 2) {
        step(c, oA);
        if (c + 1 < C) step(c + 1, oB);
    }
    // the final state, for outputs taken after the last chunk's step
    publish_state(acc, WT + ((size_t)unit * (C + 1) + C) * 2 * LD * LD, nullptr, w, lane, h, colg);
    float* We = Wend + (size_t)unit * LD * LD;
#pragma unroll
    for (int i = 0; i < 16; ++i) We[(32 * w + crow(i, h)) * LD + colg] = acc[i];
}

// ===========================================================================
// lc_chunk: Z for one (unit, chunk), fused, in sub-blocks of SB = 64 tokens.
//
// Inside a chunk every gradient is taken at W_c, so the dual-form output
//     Z = Q W_c + tril(Q K^T) Gn,     Gn = D (V - K W_c)   (= -D E)
// splits over sub-blocks i (rows i*SB .. i*SB+SB-1) by associativity:
//     Z_i = Q_i W'_i + tril(Q_i K_i^T) Gn_i,   W'_i = W_c + sum_{j<i} K_j^T Gn_j.
// W'_i is the state after the chunk's first i*SB tokens with gradients at W_c
// (the page's "accumulated weight delta", section 4 of "Test-Time Training:
// Linear Complexity Beyond Attention", taken at sub-block granularity). The
// causal product thus only spans SB keys; the rest of the sum is carried by
// W', which stays in registers as an fp32 MFMA accumulator.
//
// Wave w owns output features [32w, 32w+32) of everything (Gn, Z, W').
// Per sub-block and wave (32x32x16 bf16 MFMA, fp32 accumulation):
//   Z_m    = Q_m W'                 W' split into two bf16 terms on the fly
//   G_a    = K_a W_c                W_c^T rows of the wave held in registers
//   P_am   = K_a Q_m^T (m >= a)     the same for every wave: wave t < 3 forms
//                                   tile t and shares its two bf16 terms in LDS
//   Gn_a   = D (V_a - G_a)          two bf16 terms; V read by transpose reads
//   Z_m   += P_am^T Gn_a            P (masked on the diagonal) as two bf16 terms
//   W'    += K_a^T Gn_a             K^T by transpose reads
// The C layout of G and P (lane = column, rows 8(i/4) + 4h + i%4) is used
// directly as the B / A operand of the next product: the k index runs over
// those rows in that order, and the other operand is read to match.
// W' keeps its rows (in-features) in a permuted order: the transpose reads
// that form the A operand of its update hand row i of each 32 the feature
// sigma(i), sigma swapping bits 2 and 3, so that C slots 8s..8s+7 of lane
// half h hold the contiguous features 32r + 16s + 8h + 0..7, and the Q
// operand of Q_m W' is one 16-byte row piece.
//
// LDS: W_c^T (two terms, 64 KB; read into registers at the start, then the
// shared score tiles, 12 KB) and two buffers of K, Q, V sub-block tiles
// (48 KB each), filled by direct global->LDS loads issued one sub-block
// ahead and spread over the G products. Two barriers per sub-block (the
// tiles landed; the score tiles published). The stores of Z go out one
// after each product of the W' update, in its shadow.
// ===========================================================================
constexpr int SB = 64;                  // tokens per sub-block

__shared__ __attribute__((aligned(16))) uint16_t lc_wc[2 * LD * LD];    // W_c^T [term][n][k]
__shared__ __attribute__((aligned(16))) uint16_t lc_buf0[3 * SB * LD];  // K, Q, V of even sub-blocks
__shared__ __attribute__((aligned(16))) uint16_t lc_buf1[3 * SB * LD];  // K, Q, V of odd sub-blocks

// Direct loads of 256-byte rows from `src` (row-major, LD bf16 per row) into a
// swizzled LDS tile: 1 KB (4 rows) per wave instruction, PER_WAVE instructions
// per wave; w must be wave-uniform.
template <int PER_WAVE>
__device__ __forceinline__ void rows_dma(char* dst, const uint16_t* src, int w, int lane)
{
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
        const int ins = PER_WAVE * w + k;
        const int sl = ins * 64 + lane;
        const int r = sl >> 4, p = (sl & 15) ^ rsw(r);
        dma16(src + (size_t)r * LD + p * 8, __builtin_amdgcn_readfirstlane(lds_addr(dst + ins * 1024)));
    }
}

// K, Q, V rows [t, t + SB) of the unit into one buffer (3 x 16 KB).
__device__ __forceinline__ void sub_dma(uint16_t* buf, const uint16_t* Ku, const uint16_t* Qu, const uint16_t* Vu,
                                        int t, int w, int lane)
{
    char* b = reinterpret_cast<char*>(buf);
    rows_dma<4>(b, Ku + (size_t)t * LD, w, lane);
    rows_dma<4>(b + SB * LD * 2, Qu + (size_t)t * LD, w, lane);
    rows_dma<4>(b + 2 * SB * LD * 2, Vu + (size_t)t * LD, w, lane);
}

// One of the 12 direct-load instructions of sub_dma (J = 4 * tensor + k).
template <int J>
__device__ __forceinline__ void sub_dma_one(uint16_t* buf, const uint16_t* Ku, const uint16_t* Qu, const uint16_t* Vu,
                                            int t, int w, int lane)
{
    constexpr int T = J / 4, k = J % 4;
    const uint16_t* src = (T == 0 ? Ku : T == 1 ? Qu : Vu) + (size_t)t * LD;
    char* dst = reinterpret_cast<char*>(buf) + T * SB * LD * 2;
    const int ins = 4 * w + k;
    const int sl = ins * 64 + lane;
    const int r = sl >> 4, p = (sl & 15) ^ rsw(r);
    dma16(src + (size_t)r * LD + p * 8, __builtin_amdgcn_readfirstlane(lds_addr(dst + ins * 1024)));
}

// Row read: piece p of row r (16 bytes).
__device__ __forceinline__ bf16x8 ld_piece(const char* tile, int r, int p)
{
    return *reinterpret_cast<const bf16x8*>(tile + swz(r, p));
}

// Transpose read: lane gets rows row0 + 4h + 0..3 of column col0 + lane % 32.
__device__ __forceinline__ uint2 ld_tr4(const char* tile, int row0, int col0, int lane)
{
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const int q = lane >> 4, r16 = lane & 15;
    const int row = row0 + 4 * (q >> 1) + (r16 >> 2);
    const int col = col0 + 16 * (q & 1) + 4 * (r16 & 3);
    const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(tile + swz(row, col >> 3) + (col & 7) * 2));
    return __builtin_bit_cast(uint2, v);
}

// As ld_tr4, with the two middle 4-column segments of each 16 swapped: lane
// (feature) slot c of the result holds column sigma(c), sigma swapping bits 2 and 3.
__device__ __forceinline__ uint2 ld_tr4s(const char* tile, int row0, int col0, int lane)
{
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const int q = lane >> 4, r16 = lane & 15;
    const int row = row0 + 4 * (q >> 1) + (r16 >> 2);
    const int col = col0 + 16 * (q & 1) + 4 * (((r16 & 1) << 1) | ((r16 >> 1) & 1));
    const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(tile + swz(row, col >> 3) + (col & 7) * 2));
    return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ bf16x8 cat8(uint2 a, uint2 b)
{
    return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// Eight fp32 values (C slots 8s .. 8s+7) as two bf16 operand terms, optionally
// masked to the causal part of a diagonal tile (key row <= query column).
__device__ __forceinline__ void pack_p(const f32x16& p, int s, bool diag, int h, int l32, bf16x8 (&out)[2])
{
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int i = 8 * s + j;
        x[j] = (!diag || crow(i, h) <= l32) ? p[i] : 0.f;
    }
    terms8<2>(x, out);
}

struct ChunkCtx {
    const uint16_t *Ku, *Qu, *Vu;
    const float* etau;                  // per-token eta of the unit, or null
    float two_eta;                      // 2 eta_const
    __amdgpu_buffer_rsrc_t zr;          // Z rows of the unit (buffer stores: uniform row offsets)
    int c0, nsb, w, lane, h, l32;
};

// Two bf16 terms of Gn = D (V - G) for one 32-token tile (C layout of G:
// column = feature 32w + l32, rows = tokens 32a + crow(e, h)), per k-step s.
template <bool PER_TOKEN>
__device__ __forceinline__ void grad_terms(const ChunkCtx& x, const char* vt, int i, int a, const f32x16& g,
                                           bf16x8 (&gnb)[2][2])
{
    float gn[16];
#pragma unroll
    for (int mq = 0; mq < 4; ++mq) {
        const uint2 vv = ld_tr4(vt, 32 * a + 8 * mq, 32 * x.w, x.lane);
        const float v4[4] = {__builtin_bit_cast(float, vv.x << 16), __builtin_bit_cast(float, vv.x & 0xFFFF0000u),
                             __builtin_bit_cast(float, vv.y << 16), __builtin_bit_cast(float, vv.y & 0xFFFF0000u)};
        float d4[4] = {x.two_eta, x.two_eta, x.two_eta, x.two_eta};
        if constexpr (PER_TOKEN) {
            const float4 e4 = *reinterpret_cast<const float4*>(x.etau + x.c0 + i * SB + 32 * a + 8 * mq + 4 * x.h);
            d4[0] = 2.f * e4.x;
            d4[1] = 2.f * e4.y;
            d4[2] = 2.f * e4.z;
            d4[3] = 2.f * e4.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) gn[4 * mq + e] = d4[e] * (v4[e] - g[4 * mq + e]);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        float xv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = gn[8 * s + j];
        terms8<2>(xv, gnb[s]);
    }
}


template <bool PER_TOKEN>
__device__ __forceinline__ void chunk_step(const ChunkCtx& x, uint16_t* cur, uint16_t* nxt, int i, f32x16 (&accW)[4],
                                           const bf16x8 (&wreg)[LD / 16][2])
{
    const int w = x.w, lane = x.lane, h = x.h, l32 = x.l32;
    // this wave's loads into `cur` (and its Z stores) are done; after the
    // barrier every wave's are, and no wave still reads `nxt`
    __builtin_amdgcn_s_waitcnt(0x0070);                  // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // next sub-block (the last one reloads itself into the idle buffer)
    const int tn = x.c0 + min(i + 1, x.nsb - 1) * SB;

    const char* kt = reinterpret_cast<const char*>(cur);
    const char* qt = kt + SB * LD * 2;
    const char* vt = kt + 2 * SB * LD * 2;

    // ---- G_a = K_a W_c for both token tiles (two terms of W_c), then the
    // three causal score tiles P^T_am = K_a Q_m^T; operands one k-step ahead
    f32x16 g0 = {}, g1 = {};
    {
        bf16x8 k0 = ld_piece(kt, l32, h), k1 = ld_piece(kt, 32 + l32, h);
#pragma unroll
        for (int ks = 0; ks < LD / 16; ++ks) {
            bf16x8 k0n = k0, k1n = k1;
            if (ks + 1 < LD / 16) {
                k0n = ld_piece(kt, l32, 2 * ks + 2 + h);
                k1n = ld_piece(kt, 32 + l32, 2 * ks + 2 + h);
            }
            g0 = mfma_32x32x16(k0, wreg[ks][1], g0);
            g1 = mfma_32x32x16(k1, wreg[ks][1], g1);
            g0 = mfma_32x32x16(k0, wreg[ks][0], g0);
            g1 = mfma_32x32x16(k1, wreg[ks][0], g1);
            k0 = k0n; k1 = k1n;
            SCHED_GROUP(SG_DS_R, 2);
            SCHED_GROUP(SG_MFMA, 4);
            __builtin_amdgcn_sched_barrier(0);
            // the next sub-block's direct loads, spread over the product
            switch (ks) {
            case 0: sub_dma_one<0>(nxt, x.Ku, x.Qu, x.Vu, tn, w, lane); sub_dma_one<8>(nxt, x.Ku, x.Qu, x.Vu, tn, w, lane); break;
            case 1: sub_dma_one<1>(nxt, x.Ku, x.Qu, x.Vu, tn, w, lane); break;
            case 2: sub_dma_one<2>(nxt, x.Ku, x.Qu, x.Vu, tn, w, lane); sub_dma_one<9>(nxt, x.Ku, x.Qu, x.Vu, tn, w, lane); break;
            case 3: sub_dma_one<3>(nxt, x.Ku, x.Qu, x.Vu, tn, w, lane); break;
            case 4: sub_dma_one<4>(nxt, x.Ku, x.Qu, x.Vu, tn, w, lane); sub_dma_one<10>(nxt, x.Ku, x.Qu, x.Vu, tn, w, lane); break;
            case 5: sub_dma_one<5>(nxt, x.Ku, x.Qu, x.Vu, tn, w, lane); break;
            case 6: sub_dma_one<6>(nxt, x.Ku, x.Qu, x.Vu, tn, w, lane); sub_dma_one<11>(nxt, x.Ku, x.Qu, x.Vu, tn, w, lane); break;
            default: sub_dma_one<7>(nxt, x.Ku, x.Qu, x.Vu, tn, w, lane); break;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // The three causal score tiles P^T_am = K_a Q_m^T, (a, m) = (0, 0), (0, 1),
    // (1, 1), are the same for every wave: wave w < 3 computes tile w and
    // publishes its two bf16 terms in LDS (the W_c^T region, free once the
    // state is in registers), from where every wave reads all three.
    f32x16 pt = {};
    if (w < 3) {
        const int a = (w == 2) ? 1 : 0, m = (w == 0) ? 0 : 1;
        bf16x8 kx = ld_piece(kt, 32 * a + l32, h), qx = ld_piece(qt, 32 * m + l32, h);
#pragma unroll
        for (int ks = 0; ks < LD / 16; ++ks) {
            bf16x8 kxn = kx, qxn = qx;
            if (ks + 1 < LD / 16) {
                kxn = ld_piece(kt, 32 * a + l32, 2 * ks + 2 + h);
                qxn = ld_piece(qt, 32 * m + l32, 2 * ks + 2 + h);
            }
            pt = mfma_32x32x16(kx, qx, pt);
            kx = kxn; qx = qxn;
        }
    }
    // Gn_a = D (V_a - G_a) as two bf16 terms
    bf16x8 gnb[2][2][2];                                 // [a][s][term]
    grad_terms<PER_TOKEN>(x, vt, i, 0, g0, gnb[0]);
    grad_terms<PER_TOKEN>(x, vt, i, 1, g1, gnb[1]);
    bf16x8 (*pshare)[2][2][64] = reinterpret_cast<bf16x8 (*)[2][2][64]>(lc_wc);   // [tile][s][term][lane]
    if (w < 3) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 pp[2];
            pack_p(pt, s, w != 1, h, l32, pp);
            pshare[w][s][0][lane] = pp[0];
            pshare[w][s][1][lane] = pp[1];
        }
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);

    // ---- Z_m = Q_m W' + P_am^T Gn_a ; W' as B operand: k = in-features
    // 32r + crow(8s + j, h), split into two bf16 terms on the fly
    bf16x8 pa00[2][2], pa01[2][2], pa11[2][2];           // [s][term]
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            pa00[s][t] = pshare[0][s][t][lane];
            pa01[s][t] = pshare[1][s][t][lane];
            pa11[s][t] = pshare[2][s][t][lane];
        }
    f32x16 zacc[2] = {f32x16{}, f32x16{}};
    // k-block it = 2r + s: Q piece 2 it + h and the matching eight W' slots split
    // into two bf16 terms. Operands of block it + 1 are read and split while the
    // products of block it run.
    auto w_ops = [&](int it, bf16x8 (&wb)[2]) {
        const int r = it >> 1, s = it & 1;
        float xv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = accW[r][8 * s + j];
        terms8<2>(xv, wb);
    };
    {
        bf16x8 qa[2], wb[2];
        qa[0] = ld_piece(qt, l32, h);
        qa[1] = ld_piece(qt, 32 + l32, h);
        w_ops(0, wb);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            bf16x8 qn[2], wn[2];
            if (it + 1 < 8) {
                qn[0] = ld_piece(qt, l32, 2 * it + 2 + h);
                qn[1] = ld_piece(qt, 32 + l32, 2 * it + 2 + h);
                w_ops(it + 1, wn);
            }
            zacc[0] = mfma_32x32x16(qa[0], wb[1], zacc[0]);
            zacc[1] = mfma_32x32x16(qa[1], wb[1], zacc[1]);
            zacc[0] = mfma_32x32x16(qa[0], wb[0], zacc[0]);
            zacc[1] = mfma_32x32x16(qa[1], wb[0], zacc[1]);
            if (it + 1 < 8) {
                qa[0] = qn[0]; qa[1] = qn[1];
                wb[0] = wn[0]; wb[1] = wn[1];
            }
        }
    }
    // causal pairs (0,0), (0,1), (1,1); two terms each, the pair (lo, lo) dropped
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        zacc[0] = mfma_32x32x16(pa00[s][1], gnb[0][s][0], zacc[0]);
        zacc[1] = mfma_32x32x16(pa01[s][1], gnb[0][s][0], zacc[1]);
        zacc[0] = mfma_32x32x16(pa00[s][0], gnb[0][s][1], zacc[0]);
        zacc[1] = mfma_32x32x16(pa01[s][0], gnb[0][s][1], zacc[1]);
        zacc[0] = mfma_32x32x16(pa00[s][0], gnb[0][s][0], zacc[0]);
        zacc[1] = mfma_32x32x16(pa01[s][0], gnb[0][s][0], zacc[1]);
        zacc[1] = mfma_32x32x16(pa11[s][1], gnb[1][s][0], zacc[1]);
        zacc[1] = mfma_32x32x16(pa11[s][0], gnb[1][s][1], zacc[1]);
        zacc[1] = mfma_32x32x16(pa11[s][0], gnb[1][s][0], zacc[1]);
    }
    SCHED_GROUP(SG_DS_R, 14);                            // the shared score tiles, Q of block 0
    SCHED_GROUP(SG_VALU, 24);                            // W' slots of block 0
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        if (it + 1 < 8) SCHED_GROUP(SG_DS_R, 2);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            SCHED_GROUP(SG_MFMA, 1);
            if (it + 1 < 8) SCHED_GROUP(SG_VALU, 6);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- W' += K_a^T Gn_a ; A = K^T rows 32r + sigma(l32), k = tokens 32a + crow(8s + j, h).
    // The 32 stores of Z go out one after each product, in the products' shadow:
    // lane stores column 32w + l32 of row crow(e, h) of tile m, the row offset
    // split into a uniform part (8 (e / 4) rows) and an immediate (e % 4 rows).
    const int voff = ((4 * h) * LD + 32 * w + l32) * 4;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 ka[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ka[r] = cat8(ld_tr4s(kt, 32 * a + 16 * s, 32 * r, lane), ld_tr4s(kt, 32 * a + 16 * s + 8, 32 * r, lane));
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int r = jj & 3;
                accW[r] = mfma_32x32x16(ka[r], gnb[a][s][jj < 4 ? 1 : 0], accW[r]);
                __builtin_amdgcn_sched_barrier(0);
                const int idx = 16 * a + 8 * s + jj, m = idx >> 4, e = idx & 15;
                const int srow = __builtin_amdgcn_readfirstlane(x.c0 + i * SB + 32 * m + 8 * (e >> 2));
                const float v = zacc[m][e];
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), x.zr, voff + (e & 3) * LD * 4,
                                                      srow * LD * 4, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
}

template <bool PER_TOKEN>
__global__ void __launch_bounds__(LT)
lc_chunk_kernel(int N, int b, const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                const uint16_t* __restrict__ Vg, const float* __restrict__ etag, float eta_const,
                const uint16_t* __restrict__ WT, float* __restrict__ Zg)
{
    const int C = (N + b - 1) / b;
    const int unit = blockIdx.x / C, c = blockIdx.x % C;
    ChunkCtx x;
    x.c0 = c * b;
    x.nsb = min(b, N - x.c0) / SB;                       // even: chunks hold a multiple of 128 tokens
    x.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    x.lane = threadIdx.x & 63;
    x.h = x.lane >> 5;
    x.l32 = x.lane & 31;
    x.Ku = Kg + (size_t)unit * N * LD;
    x.Qu = Qg + (size_t)unit * N * LD;
    x.Vu = Vg + (size_t)unit * N * LD;
    x.etau = PER_TOKEN ? etag + (size_t)unit * N : nullptr;
    x.two_eta = 2.f * eta_const;
    x.zr = __builtin_amdgcn_make_buffer_rsrc(Zg + (size_t)unit * N * LD, (short)0, N * LD * 4, 0x00020000);

    // W_c^T (both terms, 512 rows of 256 B) and the first sub-block
    rows_dma<16>(reinterpret_cast<char*>(lc_wc), WT + ((size_t)unit * (C + 1) + c) * 2 * LD * LD, x.w, x.lane);
    sub_dma(lc_buf0, x.Ku, x.Qu, x.Vu, x.c0, x.w, x.lane);
    __builtin_amdgcn_s_waitcnt(0x0070);                  // vmcnt(0) lgkmcnt(0)
    __syncthreads();

    // W' = W_c in fp32 (hi + lo), C layout: column = output feature 32w + l32;
    // slot 4mq + e of accW[r] = in-feature 32r + 16(mq / 2) + 8h + 4(mq % 2) + e
    // (row order permuted by sigma, as the W' update's transpose reads give it)
    f32x16 accW[4];
    {
        const char* wc = reinterpret_cast<const char*>(lc_wc);
        const int n = 32 * x.w + x.l32;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int mq = 0; mq < 4; ++mq) {
                const int k0 = 32 * r + 16 * (mq >> 1) + 8 * x.h + 4 * (mq & 1);
                const int off = swz(n, k0 >> 3) + (k0 & 7) * 2;
                const uint2 hi = *reinterpret_cast<const uint2*>(wc + off);
                const uint2 lo = *reinterpret_cast<const uint2*>(wc + LD * LD * 2 + off);
                const uint32_t hv[4] = {hi.x << 16, hi.x & 0xFFFF0000u, hi.y << 16, hi.y & 0xFFFF0000u};
                const uint32_t lv[4] = {lo.x << 16, lo.x & 0xFFFF0000u, lo.y << 16, lo.y & 0xFFFF0000u};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    accW[r][4 * mq + e] = __builtin_bit_cast(float, hv[e]) + __builtin_bit_cast(float, lv[e]);
            }
    }

    // this wave's rows of W_c^T (both terms) as the B operand of G = K W_c, held
    // in registers for the whole chunk
    bf16x8 wreg[LD / 16][2];
    {
        const char* wc = reinterpret_cast<const char*>(lc_wc);
        const int wrow = 32 * x.w + x.l32;
#pragma unroll
        for (int ks = 0; ks < LD / 16; ++ks) {
            wreg[ks][0] = ld_piece(wc, wrow, 2 * ks + x.h);
            wreg[ks][1] = ld_piece(wc + LD * LD * 2, wrow, 2 * ks + x.h);
        }
    }
    for (int i = 0; i < x.nsb; i += 2) {
        chunk_step<PER_TOKEN>(x, lc_buf0, lc_buf1, i, accW, wreg);
        chunk_step<PER_TOKEN>(x, lc_buf1, lc_buf0, i + 1, accW, wreg);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);                  // the last reload lands before the LDS is released
}

// ===========================================================================
// lc_apply: block-causal outputs, Z_c = Q_c W_c (AFTER = false: the chunk's
// starting weights) or Q_c W_{c+1} (AFTER = true: the weights after its step),
// with no causal term inside the chunk. One workgroup per (unit, chunk), so the
// weights are read once per chunk; wave w computes output features
// [32w, 32w+32) with W^T rows (two bf16 terms) held as B operands in
// registers. Q streams through LDS in 64-token tiles by direct loads, one tile
// ahead.
// ===========================================================================
__shared__ __attribute__((aligned(16))) uint16_t lc_qbuf[2][SB * LD];

template <bool AFTER>
__global__ void __launch_bounds__(LT)
lc_apply_kernel(int N, int b, const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ WT,
                float* __restrict__ Zg)
{
    const int C = (N + b - 1) / b;
    const int unit = blockIdx.x / C, c = blockIdx.x % C;
    const int c0 = c * b, nsb = min(b, N - c0) / SB;
    const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint16_t* wt = WT + ((size_t)unit * (C + 1) + c + (AFTER ? 1 : 0)) * 2 * LD * LD;
    const uint16_t* Qu = Qg + (size_t)unit * N * LD;
    const __amdgpu_buffer_rsrc_t zr =
        __builtin_amdgcn_make_buffer_rsrc(Zg + (size_t)unit * N * LD, (short)0, N * LD * 4, 0x00020000);

    rows_dma<4>(reinterpret_cast<char*>(lc_qbuf[0]), Qu + (size_t)c0 * LD, w, lane);
    bf16x8 wb[LD / 16][2];
#pragma unroll
    for (int ks = 0; ks < LD / 16; ++ks)
#pragma unroll
        for (int term = 0; term < 2; ++term)
            wb[ks][term] = *reinterpret_cast<const bf16x8*>(wt + (size_t)term * LD * LD +
                                                            (size_t)(32 * w + l32) * LD + 16 * ks + 8 * h);
    const int voff = ((4 * h) * LD + 32 * w + l32) * 4;
    for (int i = 0; i < nsb; ++i) {
        __builtin_amdgcn_s_waitcnt(0x0070);              // this wave's loads of tile i (and stores) are done
        __syncthreads();                                 // tile i landed everywhere; tile i-1 no longer read
        if (i + 1 < nsb)
            rows_dma<4>(reinterpret_cast<char*>(lc_qbuf[(i + 1) & 1]), Qu + (size_t)(c0 + (i + 1) * SB) * LD, w,
                        lane);
        const char* qt = reinterpret_cast<const char*>(lc_qbuf[i & 1]);
        f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int ks = 0; ks < LD / 16; ++ks) {
            const bf16x8 q0 = ld_piece(qt, l32, 2 * ks + h);
            const bf16x8 q1 = ld_piece(qt, 32 + l32, 2 * ks + h);
            acc[0] = mfma_32x32x16(q0, wb[ks][1], acc[0]);
            acc[1] = mfma_32x32x16(q1, wb[ks][1], acc[1]);
            acc[0] = mfma_32x32x16(q0, wb[ks][0], acc[0]);
            acc[1] = mfma_32x32x16(q1, wb[ks][0], acc[1]);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int srow = __builtin_amdgcn_readfirstlane(c0 + i * SB + 32 * m + 8 * (e >> 2));
                const float v = acc[m][e];
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), zr, voff + (e & 3) * LD * 4,
                                                      srow * LD * 4, 0);
            }
    }
}

}  // namespace

size_t large_chunk_workspace_bytes(int B, int H, int N, int d, int b)
{
    if (d != LD || b % TB != 0 || N % TB != 0) return 0;
    return lc_layout(B * H, N, b).total;
}

hipError_t launch_large_chunk_linear(const LinearArgs& a, int outputs, hipStream_t stream)
{
    const int units = a.B * a.H;
    const int C = (a.N + a.b - 1) / a.b;
    const LcLayout L = lc_layout(units, a.N, a.b);
    char* ws = static_cast<char*>(a.workspace);
    uint16_t* M = reinterpret_cast<uint16_t*>(ws + L.m_off);
    float* Bm = reinterpret_cast<float*>(ws + L.b_off);
    uint16_t* WT = reinterpret_cast<uint16_t*>(ws + L.wt_off);
    const uint16_t* Q = static_cast<const uint16_t*>(a.Q);
    const uint16_t* K = static_cast<const uint16_t*>(a.K);
    const uint16_t* V = static_cast<const uint16_t*>(a.V);
    const bool per_token = a.eta != nullptr;

    if (per_token)
        hipLaunchKernelGGL((lc_gram_kernel<true>), dim3(units * C), dim3(LT), 0, stream, a.N, a.b, K, V, a.eta,
                           a.eta_const, M, Bm);
    else
        hipLaunchKernelGGL((lc_gram_kernel<false>), dim3(units * C), dim3(LT), 0, stream, a.N, a.b, K, V, a.eta,
                           a.eta_const, M, Bm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lc_scan_kernel, dim3(units * 4), dim3(LT), 0, stream, a.N, a.b, a.W0, M, Bm, WT, a.W_end);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (outputs == LC_OUT_BEFORE)
        hipLaunchKernelGGL((lc_apply_kernel<false>), dim3(units * C), dim3(LT), 0, stream, a.N, a.b, Q, WT, a.Z);
    else if (outputs == LC_OUT_AFTER)
        hipLaunchKernelGGL((lc_apply_kernel<true>), dim3(units * C), dim3(LT), 0, stream, a.N, a.b, Q, WT, a.Z);
    else if (per_token)
        hipLaunchKernelGGL((lc_chunk_kernel<true>), dim3(units * C), dim3(LT), 0, stream, a.N, a.b, Q, K, V, a.eta,
                           a.eta_const, WT, a.Z);
    else
        hipLaunchKernelGGL((lc_chunk_kernel<false>), dim3(units * C), dim3(LT), 0, stream, a.N, a.b, Q, K, V, a.eta,
                           a.eta_const, WT, a.Z);
    return hipGetLastError();
}

}  // namespace ttt
