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
// D = diag(2 eta). The path runs four kernels on one stream:
//   lc_gram : M_c and B_c for every (unit, chunk) at once (no dependence on W);
//   lc_scan : the 16-step recurrence W_c -> W_{c+1} (one workgroup per
//             (unit, 32-column block)); writes every W_c^T as two bf16 terms;
//   lc_grad : Gneg = -D (K W_c - V) per chunk, stored fp16 [token][feature];
//   lc_out  : Z = Q W_c - tril(Q K^T) diag(...) E in 128x128 blocks: for every
//             query block, the causal key blocks j <= i of its chunk.
// Workspace (caller-provided): M, B (fp32), W_c^T terms (bf16), Gneg (fp16).
//
// Precision: every product involving the fp32 state uses two bf16 terms (16
// significant bits). The causal term tril(Q K^T) Gneg takes single fp16
// operands for P = Q K^T and Gneg (11 significant bits, eight times finer than
// bf16, at the same MFMA rate); this requires |q.k| and |2 eta (k W - v)| to
// stay below the fp16 range (6.5e4), e.g. L2-normalised keys.
//
// MFMA v_mfma_f32_32x32x16_bf16 throughout. Token-major operands (the token
// index contracted in K^T K, K^T V) are read from row-major LDS tiles with the
// gfx950 transpose read ds_read_b64_tr_b16.
#include "device_common.h"
#include "kernels.h"

namespace ttt {
namespace {

constexpr int LD = 128;          // head dim of this path
constexpr int LT = 256;          // threads per workgroup
constexpr int TB = 128;          // token block of lc_grad / lc_out

// Row of a 32x32 C-layout tile held by lane half h = lane / 32 at slot i.
__device__ __forceinline__ int crow(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

struct LcLayout {
    size_t m_off, b_off, wt_off, g_off, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline LcLayout lc_layout(int units, int N, int b)
{
    const size_t C = (size_t)((N + b - 1) / b);
    LcLayout L;
    L.m_off = 0;
    L.b_off = align256(L.m_off + (size_t)units * C * LD * LD * 4);
    L.wt_off = align256(L.b_off + (size_t)units * C * LD * LD * 4);
    L.g_off = align256(L.wt_off + (size_t)units * C * 2 * LD * LD * 2);
    L.total = align256(L.g_off + (size_t)units * N * LD * 2);
    return L;
}

__device__ __forceinline__ uint32_t f16_bits_f(float x) { return pack_f16x2(x, 0.f) & 0xFFFFu; }

// ===========================================================================
// lc_gram: M_c = K^T D K (symmetric: upper 32x32 tiles computed, mirrored on
// store) and B_c = K^T D V for one (unit, chunk) per workgroup.
// ===========================================================================
constexpr int GR_TOK = 64;              // tokens per LDS stage
typedef __attribute__((address_space(3))) void lds_void;

// byte offset of piece p (16 B) of row r in a 256-byte-row tile whose pieces
// are XOR-swizzled (piece p of row r at slot p ^ (r % 16))
__device__ __forceinline__ int swz(int r, int p) { return r * 256 + ((p ^ (r & 15)) << 4); }

struct GramSmem {
    uint16_t k[2][GR_TOK * LD];         // [token][feature], swizzled pieces
    uint16_t v[2][GR_TOK * LD];
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
        const int r = sl >> 4, p = (sl & 15) ^ (r & 15);
        const size_t off = (size_t)(s * GR_TOK + r) * LD + p * 8;
        __builtin_amdgcn_global_load_lds(Ku + off, (lds_void*)(reinterpret_cast<char*>(sm.k[buf]) + (4 * w + k) * 1024),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(Vu + off, (lds_void*)(reinterpret_cast<char*>(sm.v[buf]) + (4 * w + k) * 1024),
                                         16, 0, 0);
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

// The 10 upper tiles of M and the 16 tiles of B, spread over 4 waves.
__device__ __constant__ const int kGramM[4][3][2] = {
    {{0, 0}, {0, 1}, {0, 2}}, {{0, 3}, {1, 1}, {1, 2}}, {{1, 3}, {2, 2}, {-1, -1}}, {{2, 3}, {3, 3}, {-1, -1}}};

template <bool PER_TOKEN>
__global__ void __launch_bounds__(LT)
lc_gram_kernel(int N, int b, const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
               const float* __restrict__ etag, float eta_const, float* __restrict__ Mout,
               float* __restrict__ Bout)
{
    constexpr int TA = PER_TOKEN ? 2 : 1;    // terms of the D-scaled operand
    __shared__ GramSmem sm;
    const int C = (N + b - 1) / b;
    const int unit = blockIdx.x / C, c = blockIdx.x % C;
    const int c0 = c * b, nt = min(b, N - c0);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const uint16_t* Ku = Kg + ((size_t)unit * N + c0) * LD;
    const uint16_t* Vu = Vg + ((size_t)unit * N + c0) * LD;
    const float* etau = PER_TOKEN ? etag + (size_t)unit * N + c0 : nullptr;

    // wave w: B row tile w (4 tiles) + up to 3 upper M tiles
    f32x16 accB[4], accM[3];
#pragma unroll
    for (int t = 0; t < 4; ++t) accB[t] = f32x16{};
#pragma unroll
    for (int t = 0; t < 3; ++t) accM[t] = f32x16{};

    const int nstage = nt / GR_TOK;
    gram_dma(sm, 0, 0, w, lane, Ku, Vu);
    for (int s = 0; s < nstage; ++s) {
        const int buf = s & 1;
        __syncthreads();                                 // stage s landed; stage s-1 consumed
        if (s + 1 < nstage) gram_dma(sm, buf ^ 1, s + 1, w, lane, Ku, Vu);
        const uint16_t* kt = sm.k[buf];
        const uint16_t* vt = sm.v[buf];
#pragma unroll
        for (int ks = 0; ks < GR_TOK / 16; ++ks) {
            const float* er = PER_TOKEN ? etau + s * GR_TOK + 16 * ks + 8 * h : nullptr;
            bf16x8 aw[TA];
            scaled_frag<PER_TOKEN, TA>(tok_major_frag(kt, 16 * ks, w, lane), er, aw);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x8 bv = tok_major_frag(vt, 16 * ks, t, lane);
#pragma unroll
                for (int s2 = TA - 1; s2 >= 0; --s2) accB[t] = mfma_32x32x16(aw[s2], bv, accB[t]);
            }
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const int r = kGramM[w][t][0], cc = kGramM[w][t][1];
                if (r >= 0) {
                    bf16x8 ar[TA];
                    scaled_frag<PER_TOKEN, TA>(tok_major_frag(kt, 16 * ks, r, lane), er, ar);
                    const bf16x8 bk = tok_major_frag(kt, 16 * ks, cc, lane);
#pragma unroll
                    for (int s2 = TA - 1; s2 >= 0; --s2) accM[t] = mfma_32x32x16(ar[s2], bk, accM[t]);
                }
            }
        }
    }

    const float scale = PER_TOKEN ? 1.f : 2.f * eta_const;
    const size_t base = ((size_t)unit * C + c) * LD * LD;
    float* Mo = Mout + base;
    float* Bo = Bout + base;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) Bo[(32 * w + crow(i, h)) * LD + 32 * t + l32] = scale * accB[t][i];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        const int r = kGramM[w][t][0], cc = kGramM[w][t][1];
        if (r >= 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float v = scale * accM[t][i];
                Mo[(32 * r + crow(i, h)) * LD + 32 * cc + l32] = v;
                if (r != cc) Mo[(32 * cc + l32) * LD + 32 * r + crow(i, h)] = v;
            }
        }
    }
}

// ===========================================================================
// lc_scan: W_{c+1} = W_c - M_c W_c + B_c for one (unit, 32-column block).
// Wave w holds rows [32w, 32w+32) of the block as one 32x32 C tile.
// ===========================================================================
constexpr int SC_STRIDE = LD + 4;   // floats per column of the column-major LDS block

// Operands of one scan step: this lane's A rows of M_c (row 32w + l32, the
// 8 k values of each k-step) and its 16 entries of B_c in the C layout.
__device__ __forceinline__ void scan_load(const float* Mg, const float* Bg, int unit, int C, int c, int w, int l32,
                                          int h, int colg, float4 (&ma)[LD / 16][2], float (&bv)[16])
{
    const float* Mc = Mg + ((size_t)unit * C + c) * LD * LD;
    const float* Bc = Bg + ((size_t)unit * C + c) * LD * LD;
#pragma unroll
    for (int ks = 0; ks < LD / 16; ++ks) {
        ma[ks][0] = *reinterpret_cast<const float4*>(Mc + (size_t)(32 * w + l32) * LD + 16 * ks + 8 * h);
        ma[ks][1] = *reinterpret_cast<const float4*>(Mc + (size_t)(32 * w + l32) * LD + 16 * ks + 8 * h + 4);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) bv[i] = Bc[(size_t)(32 * w + crow(i, h)) * LD + colg];
}

__global__ void __launch_bounds__(LT)
lc_scan_kernel(int N, int b, const float* __restrict__ W0, const float* __restrict__ Mg,
               const float* __restrict__ Bg, uint16_t* __restrict__ WT, float* __restrict__ Wend)
{
    __shared__ __attribute__((aligned(16))) float wcol[32 * SC_STRIDE];   // [column][row]
    const int C = (N + b - 1) / b;
    const int unit = blockIdx.x >> 2, cb = blockIdx.x & 3;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int colg = 32 * cb + l32;   // global column of this lane

    f32x16 acc;
    const float* W0u = W0 + (size_t)unit * LD * LD;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = W0u[(32 * w + crow(i, h)) * LD + colg];

    float4 ma[LD / 16][2];
    float bv[16];
    scan_load(Mg, Bg, unit, C, 0, w, l32, h, colg, ma, bv);
    for (int c = 0; c < C; ++c) {
        // publish W_c: column-major block in LDS, W_c^T terms in the workspace
        uint16_t* wt = WT + ((size_t)unit * C + c) * 2 * LD * LD;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
            const int row0 = 32 * w + 8 * q + 4 * h;
            *reinterpret_cast<float4*>(&wcol[l32 * SC_STRIDE + row0]) = v;
            uint32_t p01[2], p23[2];   // [term] packed bf16 pairs of rows row0, row0+1 / row0+2, row0+3
            split_pair<2>(v.x, v.y, p01);
            split_pair<2>(v.z, v.w, p23);
            // W_c^T[col][row0..row0+3], term 0 and term 1
            *reinterpret_cast<uint2*>(wt + (size_t)colg * LD + row0) = make_uint2(p01[0], p23[0]);
            *reinterpret_cast<uint2*>(wt + (size_t)LD * LD + (size_t)colg * LD + row0) =
                make_uint2(p01[1], p23[1]);
        }
        __syncthreads();
        // prefetch M_{c+1}, B_{c+1} (clamped: the last step reloads its own)
        float4 mn[LD / 16][2];
        float bn[16];
        scan_load(Mg, Bg, unit, C, min(c + 1, C - 1), w, l32, h, colg, mn, bn);
        f32x16 t = {};
#pragma unroll
        for (int ks = 0; ks < LD / 16; ++ks) {
            // A = M_c rows 32w + l32, k = 16ks + 8h + 0..7 ; B = W_c rows k, column colg
            const float4 b0 = *reinterpret_cast<const float4*>(&wcol[l32 * SC_STRIDE + 16 * ks + 8 * h]);
            const float4 b1 = *reinterpret_cast<const float4*>(&wcol[l32 * SC_STRIDE + 16 * ks + 8 * h + 4]);
            const float xa[8] = {ma[ks][0].x, ma[ks][0].y, ma[ks][0].z, ma[ks][0].w,
                                 ma[ks][1].x, ma[ks][1].y, ma[ks][1].z, ma[ks][1].w};
            const float xb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            bf16x8 ta[2], tb[2];
            terms8<2>(xa, ta);
            terms8<2>(xb, tb);
            t = mfma_32x32x16(ta[1], tb[0], t);
            t = mfma_32x32x16(ta[0], tb[1], t);
            t = mfma_32x32x16(ta[0], tb[0], t);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = (acc[i] - t[i]) + bv[i];
#pragma unroll
        for (int ks = 0; ks < LD / 16; ++ks) {
            ma[ks][0] = mn[ks][0];
            ma[ks][1] = mn[ks][1];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) bv[i] = bn[i];
        __syncthreads();   // wcol is rewritten next step
    }
    float* We = Wend + (size_t)unit * LD * LD;
#pragma unroll
    for (int i = 0; i < 16; ++i) We[(32 * w + crow(i, h)) * LD + colg] = acc[i];
}

// ===========================================================================
// lc_grad: Gneg[t][d] = -D_t (K W_c - V)[t][d] for every token of one chunk.
// One workgroup per (unit, chunk). W_c^T (two bf16 terms, 64 KB) is staged once
// in LDS by direct loads and is the A operand (wave w: output features
// [32w, 32w+32)); the B operand is K^T, i.e. K rows straight from global memory
// (four 32-token tiles per 128-token block, prefetched a block ahead). The C
// layout then holds, per lane, one token and four consecutive features, so V is
// read and Gneg written as 8-byte row segments, with no barrier in the loop.
// ===========================================================================
struct GradSmem {
    uint16_t wt[2][LD * LD];             // W_c^T [dout][din], term 0 and 1, swizzled rows
};

template <bool PER_TOKEN>
__global__ void __launch_bounds__(LT)
lc_grad_kernel(int N, int b, const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
               const float* __restrict__ etag, float eta_const, const uint16_t* __restrict__ WT,
               uint16_t* __restrict__ Gg)
{
    __shared__ GradSmem sm;
    const int C = (N + b - 1) / b;
    const int unit = blockIdx.x / C, c = blockIdx.x % C;
    const int c0 = c * b, nblk = min(b, N - c0) / TB;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const uint16_t* Ku = Kg + (size_t)unit * N * LD;
    const uint16_t* Vu = Vg + (size_t)unit * N * LD;
    const uint16_t* wt = WT + ((size_t)unit * C + c) * 2 * LD * LD;
    uint16_t* Gu = Gg + (size_t)unit * N * LD;

    // W_c^T terms: 4096 16-byte pieces, 16 wave instructions per wave
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int ins = 16 * w + k;
        const int sl = ins * 64 + lane;
        const int term = sl >> 11, rem = sl & 2047;
        const int r = rem >> 4, pc = (rem & 15) ^ (r & 15);
        __builtin_amdgcn_global_load_lds(wt + (size_t)term * LD * LD + r * LD + pc * 8,
                                         (lds_void*)(reinterpret_cast<char*>(&sm.wt[0][0]) + ins * 1024), 16, 0, 0);
    }
    // K rows of the first block (B operand, lane: token 32tt + l32)
    bf16x8 kb[4][LD / 16];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int ks = 0; ks < LD / 16; ++ks)
            kb[tt][ks] = *reinterpret_cast<const bf16x8*>(Ku + (size_t)(c0 + 32 * tt + l32) * LD + 16 * ks + 8 * h);
    __syncthreads();

    // A operands (W_c^T rows 32w + l32, two terms) stay in registers for the chunk
    const char* wtb = reinterpret_cast<const char*>(&sm.wt[0][0]);
    bf16x8 wa[LD / 16][2];
#pragma unroll
    for (int ks = 0; ks < LD / 16; ++ks) {
        wa[ks][0] = *reinterpret_cast<const bf16x8*>(wtb + swz(32 * w + l32, 2 * ks + h));
        wa[ks][1] = *reinterpret_cast<const bf16x8*>(wtb + LD * LD * 2 + swz(32 * w + l32, 2 * ks + h));
    }

    for (int blk = 0; blk < nblk; ++blk) {
        const int tb0 = c0 + blk * TB;
        const int tn = (blk + 1 < nblk) ? tb0 + TB : tb0;      // next block (clamped: unconditional loads)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            // G^T tile: rows = features 32w + crow(i,h), column = token tb0 + 32tt + l32
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < LD / 16; ++ks) {
                acc = mfma_32x32x16(wa[ks][1], kb[tt][ks], acc);
                acc = mfma_32x32x16(wa[ks][0], kb[tt][ks], acc);
            }
            const int tok = tb0 + 32 * tt + l32;
            // prefetch this tile's rows of the next block
#pragma unroll
            for (int ks = 0; ks < LD / 16; ++ks)
                kb[tt][ks] = *reinterpret_cast<const bf16x8*>(Ku + (size_t)(tn + 32 * tt + l32) * LD + 16 * ks + 8 * h);
            const float dt = 2.f * (PER_TOKEN ? etag[(size_t)unit * N + tok] : eta_const);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d0 = 32 * w + 8 * q4 + 4 * h;
                const uint2 vv = *reinterpret_cast<const uint2*>(Vu + (size_t)tok * LD + d0);
                const float v4[4] = {__builtin_bit_cast(float, vv.x << 16), __builtin_bit_cast(float, vv.x & 0xFFFF0000u),
                                     __builtin_bit_cast(float, vv.y << 16), __builtin_bit_cast(float, vv.y & 0xFFFF0000u)};
                float g[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) g[e] = -dt * (acc[4 * q4 + e] - v4[e]);
                *reinterpret_cast<uint2*>(Gu + (size_t)tok * LD + d0) =
                    make_uint2(pack_f16x2(g[0], g[1]), pack_f16x2(g[2], g[3]));
            }
        }
    }
}

// ===========================================================================
// lc_out: Z rows of one 256-query block: Z = Q W_c + sum_{key blocks j}
// mask(Q K_j^T) Gneg_j over the causal 128-key blocks of the chunk (Gneg_j
// token-major, its key-contracted B operand read with transpose reads). Wave w owns
// queries [64w, 64w+64) of the block (two 32-query tiles) and all 128 output
// features (four 32x32 C tiles per query tile), so every operand read from LDS
// feeds two MFMAs. K_j and Gneg_j^T tiles (32 KB each) are double-buffered in
// LDS and filled by direct global->LDS loads (no registers): one 16-byte piece
// per lane, 1 KB per wave instruction. Rows are 256 B; the 16 pieces of row r
// are stored XOR-swizzled (piece p at slot p ^ (r % 16)) so that 32 lanes
// reading the same piece of 32 different rows hit distinct banks.
// ===========================================================================
constexpr int QB = 256;                 // queries per lc_out workgroup

struct OutSmem {
    uint16_t k[2][TB * LD];             // K_j [key][feature], swizzled pieces
    uint16_t g[2][TB * LD];             // Gneg_j [key][feature], fp16, swizzled pieces
};


// Fill one K tile and one Gneg^T tile (key block kb) with direct LDS loads:
// wave w writes LDS pieces [(8w + k) * 64, +64) of each tile.
__device__ __forceinline__ void out_dma(OutSmem& sm, int buf, int kb, int w, int lane, int N,
                                        const uint16_t* Ku, const uint16_t* Gu)
{
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int sl = (8 * w + k) * 64 + lane;          // 16-byte slot in the tile
        const int r = sl >> 4, p = (sl & 15) ^ (r & 15); // row and the piece that lives there
        char* kdst = reinterpret_cast<char*>(sm.k[buf]) + (8 * w + k) * 1024;
        char* gdst = reinterpret_cast<char*>(sm.g[buf]) + (8 * w + k) * 1024;
        __builtin_amdgcn_global_load_lds(Ku + (size_t)(kb * TB + r) * LD + p * 8, (lds_void*)kdst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(Gu + (size_t)(kb * TB + r) * LD + p * 8, (lds_void*)gdst, 16, 0, 0);
    }
}

__global__ void __launch_bounds__(LT)
lc_out_kernel(int N, int b, const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
              const uint16_t* __restrict__ WT, const uint16_t* __restrict__ GT, float* __restrict__ Zg)
{
    __shared__ OutSmem sm;
    const int C = (N + b - 1) / b;
    const int bpc = (b + QB - 1) / QB;                   // query blocks per (full) chunk
    const int units = gridDim.x / (C * bpc);
    // heaviest blocks (largest in-chunk index, most key blocks) first
    const int unit = blockIdx.x % units;
    const int rank = blockIdx.x / units;
    const int iin = bpc - 1 - rank / C;                  // query block index inside the chunk
    const int c = rank % C;
    const int c0 = c * b;
    const int q0 = c0 + iin * QB;                        // first query of the block
    const int cend = min(c0 + b, N);                     // end of the chunk
    if (q0 >= cend) return;                              // past a short chunk
    const int nq = min(QB, cend - q0);                   // 128 or 256
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const uint16_t* Qu = Qg + (size_t)unit * N * LD;
    const uint16_t* Ku = Kg + (size_t)unit * N * LD;
    const uint16_t* Gu = GT + (size_t)unit * LD * N;
    const uint16_t* wt = WT + ((size_t)unit * C + c) * 2 * LD * LD;
    const bool active = 64 * w < nq;                     // this wave has queries
    const int qw = q0 + 64 * w;                          // first query of this wave

    // causal key blocks of the chunk visible to this query block
    const int kb0 = c0 / TB;
    const int nkb = (iin * QB + nq) / TB;
    out_dma(sm, 0, kb0, w, lane, N, Ku, Gu);

    // Q rows as operands: A of Q W_c and B of K_j Q^T share the registers
    bf16x8 qa[2][LD / 16];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int ks = 0; ks < LD / 16; ++ks) {
            const int q = active ? qw + 32 * qt + l32 : q0;
            qa[qt][ks] = *reinterpret_cast<const bf16x8*>(Qu + (size_t)q * LD + 16 * ks + 8 * h);
        }

    // Z = Q W_c  (B = W_c: row k = input feature, column n -> W_c^T row n, two terms)
    f32x16 acc[2][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        acc[0][t] = f32x16{};
        acc[1][t] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < LD / 16; ++ks) {
            const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(wt + (size_t)(32 * t + l32) * LD + 16 * ks + 8 * h);
            const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(wt + (size_t)LD * LD + (size_t)(32 * t + l32) * LD +
                                                               16 * ks + 8 * h);
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                acc[qt][t] = mfma_32x32x16(qa[qt][ks], b1, acc[qt][t]);
                acc[qt][t] = mfma_32x32x16(qa[qt][ks], b0, acc[qt][t]);
            }
        }
    }

    const int qin = iin * QB + 64 * w;                   // first query of the wave inside the chunk
    const int q16 = lane >> 4, r16 = lane & 15;          // transpose-read lane coordinates
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    for (int j = 0; j < nkb; ++j) {
        __syncthreads();                                 // tile j landed; tile j-1 consumed
        if (j + 1 < nkb) out_dma(sm, (j + 1) & 1, kb0 + j + 1, w, lane, N, Ku, Gu);
        if (!active || TB * j > qin + 63) continue;      // every key of the block is after every query
        const char* kt_base = reinterpret_cast<const char*>(sm.k[j & 1]);
        const char* gt_base = reinterpret_cast<const char*>(sm.g[j & 1]);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int kmin = TB * j + 32 * kt;           // first key of the tile inside the chunk
            if (kmin > qin + 63) continue;
            // P^T = K Q^T for 32 keys x 64 queries
            f32x16 pt[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int ks = 0; ks < LD / 16; ++ks) {
                const bf16x8 ak = *reinterpret_cast<const bf16x8*>(kt_base + swz(32 * kt + l32, 2 * ks + h));
                pt[0] = mfma_32x32x16(ak, qa[0][ks], pt[0]);
                pt[1] = mfma_32x32x16(ak, qa[1][ks], pt[1]);
            }
            const bool need_mask = kmin + 31 > qin;      // some key of the tile is after some query
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f16x8 pa[2];
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    float x[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        const int i = 8 * half + jj;
                        const bool keep = !need_mask || kmin + crow(i, h) <= qin + 32 * qt + l32;
                        x[jj] = keep ? pt[qt][i] : 0.f;
                    }
                    pa[qt] = __builtin_bit_cast(
                        f16x8, make_uint4(pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3]),
                                          pack_f16x2(x[4], x[5]), pack_f16x2(x[6], x[7])));
                }
                const int kbase = 32 * kt + 16 * half;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    // B operand: keys kbase + {4h..4h+3, 8+4h..8+4h+3} of feature 32t + l32,
                    // two transpose reads of the token-major tile
                    const int grow = kbase + 4 * h + (r16 >> 2);
                    const int gcol = 32 * t + 16 * (q16 & 1) + 4 * (r16 & 3);
                    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_bf16x4*)(gt_base + swz(grow, gcol >> 3) + (gcol & 7) * 2));
                    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_bf16x4*)(gt_base + swz(grow + 8, gcol >> 3) + (gcol & 7) * 2));
                    const uint2 ul = __builtin_bit_cast(uint2, lo), uh = __builtin_bit_cast(uint2, hi);
                    const f16x8 gb = __builtin_bit_cast(f16x8, make_uint4(ul.x, ul.y, uh.x, uh.y));
                    acc[0][t] = mfma_32x32x16_f16(pa[0], gb, acc[0][t]);
                    acc[1][t] = mfma_32x32x16_f16(pa[1], gb, acc[1][t]);
                }
            }
        }
    }

    if (!active) return;
    float* Zu = Zg + (size_t)unit * N * LD;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                Zu[(size_t)(qw + 32 * qt + crow(i, h)) * LD + 32 * t + l32] = acc[qt][t][i];
}

}  // namespace

size_t large_chunk_workspace_bytes(int B, int H, int N, int d, int b)
{
    if (d != LD || b % TB != 0 || N % TB != 0) return 0;
    return lc_layout(B * H, N, b).total;
}

hipError_t launch_large_chunk_linear(const LinearArgs& a, hipStream_t stream)
{
    const int units = a.B * a.H;
    const int C = (a.N + a.b - 1) / a.b;
    const LcLayout L = lc_layout(units, a.N, a.b);
    char* ws = static_cast<char*>(a.workspace);
    float* M = reinterpret_cast<float*>(ws + L.m_off);
    float* Bm = reinterpret_cast<float*>(ws + L.b_off);
    uint16_t* WT = reinterpret_cast<uint16_t*>(ws + L.wt_off);
    uint16_t* GT = reinterpret_cast<uint16_t*>(ws + L.g_off);
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
    if (per_token)
        hipLaunchKernelGGL((lc_grad_kernel<true>), dim3(units * C), dim3(LT), 0, stream, a.N, a.b, K, V, a.eta,
                           a.eta_const, WT, GT);
    else
        hipLaunchKernelGGL((lc_grad_kernel<false>), dim3(units * C), dim3(LT), 0, stream, a.N, a.b, K, V, a.eta,
                           a.eta_const, WT, GT);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(lc_out_kernel, dim3(units * C * ((a.b + QB - 1) / QB)), dim3(LT), 0, stream, a.N, a.b, Q,
                       K, WT, GT, a.Z);
    return hipGetLastError();
}

}  // namespace ttt
