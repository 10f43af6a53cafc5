// outer_layer.hip -- the projections and the output stage that turn the inner
// TTT-Linear model into a whole layer (page "Test-Time Training: Linear
// Complexity Beyond Attention", sections "1. The Self-Supervised Inner-Loop
// Task" and "3. Forward Evaluation and Output Projection"):
//
//     q_t = W_Q x_t,  k_t = W_K x_t / ||W_K x_t||,  v_t = W_V x_t   (per head)
//     z_t = inner model (the chunked dual form, ttt_linear_fwd's small-b path)
//     y_t = W_O (LayerNorm(z_t) + q_t)        (LayerNorm per head, own affine)
//
// Three kernels:
//  * layer_gemm_kernel<.., EPI_QKV>: [Q | K | V] = x [W_Q; W_K; W_V]^T on bf16
//    MFMA with fp32 accumulation. Each wave owns 64 tokens x 64 outputs = one
//    head of one projection, taken as the transposed tile (a lane holds
//    consecutive outputs of one token), so the key normalisation is an in-lane
//    sum plus one lane swap; Q, K, V leave head-major [B, H, N, 64] as two bf16
//    planes each (the RNE rounding, then the rounding of the remainder: 16
//    significant bits), the form in which the inner kernel consumes two-term
//    streams, staged through LDS so that every store writes whole head rows.
//  * layer_outprep_kernel: A = LayerNorm(z) * gamma_o + beta_o + q per (token,
//    head) row, written token-major as two bf16 terms (16 significant bits).
//  * layer_gemm_kernel<.., EPI_ROWS>: y = [A_hi | A_lo] [W_O | W_O]^T, i.e. the
//    two terms reduced against the same W_O rows; y leaves in fp32.
// Both GEMMs take the weight output-major ([out][in], in-features contiguous),
// so both MFMA operands are 16-byte rows of LDS tiles. The logical tile order
// keeps all output tiles of a token block on one XCD so the re-read token rows
// hit that XCD's L2.
#include "device_common.h"
#include "kernels.h"

#include <algorithm>

namespace ttt {
namespace {

constexpr int HDIM = 64;     // head width
constexpr int GT = 256;      // threads per workgroup (four waves)

// Row of a 32x32 C-layout tile held by lane half h = lane / 32 at slot i.
__device__ __forceinline__ int crow(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// ===========================================================================
// The GEMM core shared by both sides:
//     C[m][n] = sum_{k < K} A[m][k] * Bw[n][k mod KW]
// with A (bf16, row stride lda) indexed by token m = (sequence bi, token t) and
// Bw (bf16, output-major, row stride ldb). The wrap KW lets the output stage
// feed the two bf16 terms of its operand as one K = 2 * H*64 reduction
// against the same W_O rows. A workgroup computes TM tokens of one sequence x
// TN outputs with (TM/64) * (TN/64) waves, each owning a 64 x 64 block.
// Operand tiles stream global -> LDS with direct loads, 64-deep stages, NS
// stages resident (NS - 1 in flight while one is read). Both GEMMs use
// 256 x 192 tiles (twelve waves): at the layer's sizes that is a whole number
// of rounds of workgroups over the chip, and each loaded byte feeds 110 flops
// (LDS bandwidth, not the matrix cores, bounds smaller tiles here).
// ===========================================================================
constexpr int GK = 64;       // reduction depth of one LDS stage

// Tiles hold rows of 64 bf16 (128 bytes = 8 pieces, half of the 64 banks, the
// half set by r & 1); piece p of row r sits at slot p ^ ((r >> 1) & 7), so 16
// consecutive rows read at one piece start on 16 different 4-bank groups.
__device__ __forceinline__ int psw(int r, int p) { return r * 128 + ((p ^ ((r >> 1) & 7)) << 4); }

constexpr int vmcnt_imm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8); }

enum { EPI_QKV = 0, EPI_ROWS = 1 };

// Logical tile L -> (token block rt, output tile nt). Token blocks are taken in
// super-rows of GR; inside one, output tiles in groups of GC, and inside a
// group every (block, tile) pair. An XCD's contiguous range of logical tiles
// then keeps a super-row of token rows resident in its L2 while the weight
// rows stream past one group at a time, instead of the whole weight per block.
constexpr int GR = 8, GC = 3;

__device__ __forceinline__ void grouped_tile(int L, int row_tiles, int tiles_n, int& rt, int& nt)
{
    const int sr = L / (GR * tiles_n);
    const int rows = min(GR, row_tiles - sr * GR);
    const int rem = L - sr * GR * tiles_n;
    const int cg = rem / (rows * GC);
    const int cols = min(GC, tiles_n - cg * GC);
    const int rem2 = rem - cg * rows * GC;
    rt = sr * GR + rem2 / cols;
    nt = cg * GC + rem2 % cols;
}

struct GemmArgs {
    int N, H;                    // tokens per sequence, heads
    int K, KW;                   // reduction length, wrap of the weight's k index
    int n_out;                   // valid outputs (rows of the stacked weight)
    int lda, ldb;
    int tiles_t, tiles_n, total;
    const uint16_t* A;
    const uint16_t* W0;          // weight rows [0, rows_per_w), then W1, W2 (EPI_QKV)
    const uint16_t* W1;
    const uint16_t* W2;
    int rows_per_w;
    float* out0;                 // EPI_ROWS: y [tokens][n_out]
    uint16_t* qkv[3];            // EPI_QKV: Q, K, V hi planes (lo planes `plane` elements later)
    size_t plane;
};

template <int TM, int TN, int NS, int EPI>
__global__ void __launch_bounds__(TM * TN / 64)
layer_gemm_kernel(GemmArgs g)
{
    constexpr int WR = TM / 64, WC = TN / 64, NW = WR * WC;
    constexpr int NIA = TM / 8, NIB = TN / 8;              // DMA instructions per stage (1 KB = 8 rows each)
    constexpr int NI = NIA + NIB;
    constexpr int PER = (NI + NW - 1) / NW;                // ... per wave: waves w < REM issue PER,
    constexpr int REM = NI % NW;                           // the others PER - 1 (REM = 0: all PER)
    constexpr int SA = TM * GK * 2, SB = TN * GK * 2;    // stage bytes
    constexpr int SMEM = (EPI == EPI_QKV && NW * 8192 > NS * (SA + SB)) ? NW * 8192 : NS * (SA + SB);
    __shared__ __attribute__((aligned(16))) char smem[SMEM];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    const int wr = w / WC, wc = w % WC;
    const bool full = REM == 0 || w < REM;                 // this wave issues PER instructions
    const uint32_t base = lds_addr(smem);

    // Persistent (one workgroup per compute unit): a workgroup takes tiles
    // blockIdx.x, + gridDim.x, ...; no launch between tiles, and the L2 writes
    // one tile's outputs back while the next tile's products run.
    for (int L = blockIdx.x; L < g.total; L += gridDim.x) {
        int rt, nt;
        grouped_tile(xcd_tile(L, g.total), g.tiles_t * (g.total / (g.tiles_t * g.tiles_n)), g.tiles_n, rt, nt);
        const int bi = rt / g.tiles_t, t0 = (rt % g.tiles_t) * TM, n0 = nt * TN;

        // DMA instruction j of this wave covers 8 tile rows; rows past the
        // sequence or past the last output are clamped to a valid row (their
        // results are never stored).
        const uint16_t* src[PER];
        uint32_t dst[PER];
        bool isb[PER];
    #pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int ins = min(w + NW * j, NI - 1);         // (clamped for the waves that skip it)
            // with NIA a multiple of NW, whether instruction j loads the weight does not depend on w
            const bool b = (NIA % NW == 0) ? (NW * j >= NIA) : (ins >= NIA);
            const int r = (b ? ins - NIA : ins) * 8 + (lane >> 3);
            const int p = (lane & 7) ^ ((r >> 1) & 7);
            if (!b) {
                const int t = min(t0 + r, g.N - 1);
                src[j] = g.A + ((size_t)bi * g.N + t) * g.lda + p * 8;
                dst[j] = base + ins * 1024;
            } else {
                int n = min(n0 + r, g.n_out - 1);
                const uint16_t* Wt = g.W0;
                if (EPI == EPI_QKV) {
                    const int which = n / g.rows_per_w;
                    Wt = which == 0 ? g.W0 : (which == 1 ? g.W1 : g.W2);
                    n -= which * g.rows_per_w;
                }
                src[j] = Wt + (size_t)n * g.ldb + p * 8;
                dst[j] = base + NS * SA + (ins - NIA) * 1024;
            }
            isb[j] = b;
        }
        auto issue = [&](int kb, int buf) {
            const int ka = kb * GK;
            int kw = ka;
            if (kw >= g.KW) kw -= g.KW;
    #pragma unroll
            for (int j = 0; j < PER; ++j)
                if (j + 1 < PER || full)
                    dma16(src[j] + (isb[j] ? kw : ka),
                          __builtin_amdgcn_readfirstlane(dst[j] + buf * (isb[j] ? SB : SA)));
        };

        f32x16 acc[2][2];
    #pragma unroll
        for (int a = 0; a < 2; ++a)
    #pragma unroll
            for (int c = 0; c < 2; ++c)
    #pragma unroll
                for (int i = 0; i < 16; ++i) acc[a][c][i] = 0.f;

        const int KB = g.K / GK;
    #pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            if (s < KB) issue(s, s);
        for (int kb = 0; kb < KB; ++kb) {
            // stage kb has landed once at most the later stages' loads are pending
            const int later = min(KB - 1, kb + NS - 2) - kb;
            if (full) {
                if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER));
                else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            } else {
                if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (PER - 1)));
                else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER - 1));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
            __syncthreads();
            if (kb + NS - 1 < KB) issue(kb + NS - 1, (kb + NS - 1) % NS);
            const char* A = smem + (kb % NS) * SA;
            const char* Bt = smem + NS * SA + (kb % NS) * SB;
    #pragma unroll
            for (int ks = 0; ks < GK / 16; ++ks) {
                const int p = 2 * ks + h;
                bf16x8 av[2], bv[2];
    #pragma unroll
                for (int a = 0; a < 2; ++a)
                    av[a] = *reinterpret_cast<const bf16x8*>(A + psw(64 * wr + 32 * a + l32, p));
    #pragma unroll
                for (int c = 0; c < 2; ++c)
                    bv[c] = *reinterpret_cast<const bf16x8*>(Bt + psw(64 * wc + 32 * c + l32, p));
                // EPI_QKV takes the transposed tiles (rows = outputs, columns = tokens), so
                // a lane holds consecutive outputs of one token
    #pragma unroll
                for (int a = 0; a < 2; ++a)
    #pragma unroll
                    for (int c = 0; c < 2; ++c)
                        acc[a][c] = EPI == EPI_QKV ? mfma_32x32x16(bv[c], av[a], acc[a][c])
                                                   : mfma_32x32x16(av[a], bv[c], acc[a][c]);
            }
        }

        const int nw = n0 + 64 * wc;                 // this wave's first output (n_out is a multiple of 64)
        if (EPI == EPI_QKV) {
            // acc[a][c] slot 4q + j: token 64 wr + 32 a + l32 of the tile, output nw + 32 c + 8 q + 4 h + j.
            // The wave's 64 outputs are one head of one projection. Each plane of its
            // 64 x 64 block goes through an 8 KB LDS buffer of its own ([token][output],
            // 16-byte pieces swizzled by token), so that the global stores are whole
            // 128-byte head rows, eight per instruction.
            static_assert(EPI != EPI_QKV || SMEM >= NW * 8192, "the stage buffers hold the output staging");
            __syncthreads();                             // every wave is done with the stage buffers
            if (nw < g.n_out) {
            const int which = nw / g.rows_per_w, head = (nw - which * g.rows_per_w) / HDIM;
            uint16_t* ob = g.qkv[which] + ((size_t)bi * g.H + head) * (size_t)g.N * HDIM;
            // per 32-token half a: both planes of the half through the wave's 8 KB
            // (high terms at 0, low terms at 4 KB)
            char* wb = smem + w * 8192;
    #pragma unroll
            for (int a = 0; a < 2; ++a) {
                float sc = 1.f;
                if (which == 1) {
                    // k / ||k||: this lane holds 32 of the row's 64 entries, lane l ^ 32 the rest
                    float s = 0.f;
    #pragma unroll
                    for (int c = 0; c < 2; ++c)
    #pragma unroll
                        for (int i = 0; i < 16; ++i) s = fmaf(acc[a][c][i], acc[a][c][i], s);
                    s += __shfl_xor(s, 32, 64);
                    sc = s > 0.f ? 1.f / sqrtf(s) : 0.f;
                }
                const int r = l32;
    #pragma unroll
                for (int c = 0; c < 2; ++c)
    #pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        // two bf16 terms: RNE rounding, then the rounding of the remainder
                        uint32_t p01[2], p23[2];
                        split_pair<2>(acc[a][c][4 * q] * sc, acc[a][c][4 * q + 1] * sc, p01);
                        split_pair<2>(acc[a][c][4 * q + 2] * sc, acc[a][c][4 * q + 3] * sc, p23);
                        const int off = r * 128 + (((4 * c + q) ^ (r & 7)) << 4) + 8 * h;
                        *reinterpret_cast<uint2*>(wb + off) = make_uint2(p01[0], p23[0]);
                        *reinterpret_cast<uint2*>(wb + 4096 + off) = make_uint2(p01[1], p23[1]);
                    }
                // the same wave reads back (its LDS operations are ordered): lane L takes
                // piece L % 8 of token row 8 j + L / 8 of the half, in each plane
    #pragma unroll
                for (int pl = 0; pl < 2; ++pl)
    #pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int rr = 8 * j + (lane >> 3), k = lane & 7;
                        const uint4 v = *reinterpret_cast<const uint4*>(wb + 4096 * pl + rr * 128 + ((k ^ (rr & 7)) << 4));
                        const int t = t0 + 64 * wr + 32 * a + rr;
                        if (t < g.N) *reinterpret_cast<uint4*>(ob + (pl ? g.plane : 0) + (size_t)t * HDIM + 8 * k) = v;
                    }
            }
            }
        } else if (nw < g.n_out) {
    #pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int n = nw + 32 * c + l32;
                if (n >= g.n_out) continue;
    #pragma unroll
                for (int a = 0; a < 2; ++a)
    #pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int t = t0 + 64 * wr + 32 * a + crow(i, h);
                        if (t < g.N) g.out0[((size_t)bi * g.N + t) * g.n_out + n] = acc[a][c][i];
                    }
            }
        }
        __syncthreads();                                 // the LDS is free for the next tile's loads
    }
}

// ===========================================================================
// Output operand: A = LayerNorm(z) * gamma_o + beta_o + q for every (token,
// head) row, written token-major as two bf16 terms, Aext[token][0 .. H*64) =
// hi and Aext[token][H*64 .. 2*H*64) = lo. Sixteen lanes (one DPP row) own a
// row, four entries each, so the reads of z and q and the writes are
// contiguous 256- and 128-byte runs and the statistics are DPP row sums.
// ===========================================================================
constexpr int PT = 256;

__global__ void __launch_bounds__(PT)
layer_outprep_kernel(int N, int H, int rows, size_t plane, const float* __restrict__ Z,
                     const uint16_t* __restrict__ Qh,
                     const float* __restrict__ gamma_o, const float* __restrict__ beta_o, float eps,
                     uint32_t* __restrict__ Aext)
{
    const int gid = blockIdx.x * PT + threadIdx.x;
    const int row = gid >> 4, e = (gid & 15) * 4;     // row = (b*H + h)*N + t of the head-major arrays
    if (row >= rows) return;                          // whole DPP rows leave together
    const float4 z = *reinterpret_cast<const float4*>(Z + (size_t)row * HDIM + e);
    const uint2 qh = *reinterpret_cast<const uint2*>(Qh + (size_t)row * HDIM + e);
    const uint2 ql = *reinterpret_cast<const uint2*>(Qh + plane + (size_t)row * HDIM + e);
    const float4 q = make_float4(
        __builtin_bit_cast(float, qh.x << 16) + __builtin_bit_cast(float, ql.x << 16),
        __builtin_bit_cast(float, qh.x & 0xFFFF0000u) + __builtin_bit_cast(float, ql.x & 0xFFFF0000u),
        __builtin_bit_cast(float, qh.y << 16) + __builtin_bit_cast(float, ql.y << 16),
        __builtin_bit_cast(float, qh.y & 0xFFFF0000u) + __builtin_bit_cast(float, ql.y & 0xFFFF0000u));
    const int t = row % N, bh = row / N, hh = bh % H, bi = bh / H;
    const float mu = row16_sum(z.x + z.y + z.z + z.w) * (1.f / HDIM);
    const float c0 = z.x - mu, c1 = z.y - mu, c2 = z.z - mu, c3 = z.w - mu;
    const float var = row16_sum(c0 * c0 + c1 * c1 + c2 * c2 + c3 * c3) * (1.f / HDIM);
    const float rs = 1.f / sqrtf(var + eps);
    const float4 gm = *reinterpret_cast<const float4*>(gamma_o + hh * HDIM + e);
    const float4 bt = *reinterpret_cast<const float4*>(beta_o + hh * HDIM + e);
    const float a0 = fmaf(c0 * rs, gm.x, bt.x) + q.x;
    const float a1 = fmaf(c1 * rs, gm.y, bt.y) + q.y;
    const float a2 = fmaf(c2 * rs, gm.z, bt.z) + q.z;
    const float a3 = fmaf(c3 * rs, gm.w, bt.w) + q.w;
    uint32_t p01[2], p23[2];
    split_pair<2>(a0, a1, p01);
    split_pair<2>(a2, a3, p23);
    const size_t HD = (size_t)H * HDIM;
    uint32_t* dst = Aext + (((size_t)bi * N + t) * 2 * HD + (size_t)hh * HDIM + e) / 2;
    *reinterpret_cast<uint2*>(dst) = make_uint2(p01[0], p23[0]);
    *reinterpret_cast<uint2*>(dst + HD / 2) = make_uint2(p01[1], p23[1]);
}

// Tile shapes of the two GEMMs
constexpr int P_TM = 256, P_TN = 192, P_NS = 2;      // projections: 3 rounds at B 8, N 2048, D 768
constexpr int O_TM = 256, O_TN = 192, O_NS = 2;      // output projection: 1 round

// Compute units of the current device (the persistent GEMM grid), cached per device.
int device_cus()
{
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] <= 0) {
        int v = 0;
        cus[dev] = (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ? v : 256;
    }
    return cus[dev];
}

}  // namespace

size_t layer_workspace_region_bytes(int B, int N, int H)
{
    const size_t s = (size_t)B * H * N * HDIM * 4;
    return (s + 255) & ~(size_t)255;
}

hipError_t launch_layer_qkv(const LayerArgs& a, uint16_t* Qo, uint16_t* Ko, uint16_t* Vo, hipStream_t stream)
{
    GemmArgs g{};
    g.N = a.N;
    g.H = a.H;
    g.K = a.D;
    g.KW = a.D;
    g.rows_per_w = a.H * HDIM;
    g.n_out = 3 * g.rows_per_w;
    g.lda = a.D;
    g.ldb = a.D;
    g.tiles_t = (a.N + P_TM - 1) / P_TM;
    g.tiles_n = (g.n_out + P_TN - 1) / P_TN;
    g.total = a.B * g.tiles_t * g.tiles_n;
    g.A = static_cast<const uint16_t*>(a.x);
    g.W0 = static_cast<const uint16_t*>(a.Wq);
    g.W1 = static_cast<const uint16_t*>(a.Wk);
    g.W2 = static_cast<const uint16_t*>(a.Wv);
    g.qkv[0] = Qo;
    g.qkv[1] = Ko;
    g.qkv[2] = Vo;
    g.plane = (size_t)a.B * a.H * a.N * HDIM;
    hipLaunchKernelGGL((layer_gemm_kernel<P_TM, P_TN, P_NS, EPI_QKV>), dim3(std::min(g.total, device_cus())),
                       dim3(P_TM * P_TN / 64), 0,
                       stream, g);
    return hipGetLastError();
}

hipError_t launch_layer_out(const LayerArgs& a, const float* Z, const uint16_t* Qh, void* aext, hipStream_t stream)
{
    const int HD = a.H * HDIM;
    const int rows = a.B * a.H * a.N;
    const size_t threads = (size_t)rows * 16;
    hipLaunchKernelGGL(layer_outprep_kernel, dim3((unsigned)((threads + PT - 1) / PT)), dim3(PT), 0, stream, a.N,
                       a.H, rows, (size_t)a.B * a.H * a.N * HDIM, Z, Qh, a.out_gamma, a.out_beta, a.eps,
                       static_cast<uint32_t*>(aext));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    GemmArgs g{};
    g.N = a.N;
    g.H = a.H;
    g.K = 2 * HD;
    g.KW = HD;
    g.rows_per_w = a.D;
    g.n_out = a.D;
    g.lda = 2 * HD;
    g.ldb = HD;
    g.tiles_t = (a.N + O_TM - 1) / O_TM;
    g.tiles_n = (a.D + O_TN - 1) / O_TN;
    g.total = a.B * g.tiles_t * g.tiles_n;
    g.A = static_cast<const uint16_t*>(aext);
    g.W0 = static_cast<const uint16_t*>(a.Wo);
    g.out0 = a.y;
    hipLaunchKernelGGL((layer_gemm_kernel<O_TM, O_TN, O_NS, EPI_ROWS>), dim3(std::min(g.total, device_cus())),
                       dim3(O_TM * O_TN / 64), 0,
                       stream, g);
    return hipGetLastError();
}

}  // namespace ttt
