// smallb_common.h -- pieces shared by the small-b kernels (one workgroup per
// (sequence, head) unit, d = 64, chunks of at most 16 tokens): LDS staging of
// Q/K/V/eta chunks with a register prefetch ring, and MFMA operand loaders that
// turn LDS rows into bf16-term operands.
#pragma once

#include "device_common.h"

namespace ttt {
namespace smallb {

constexpr int D = 64;
constexpr int ROWS = 16;
constexpr int THREADS = 256;
constexpr int PF = 4;        // chunks of Q/K/V/eta in flight per workgroup

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
        const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        terms8<T>(x, out);
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
struct Pieces {
    static constexpr int PIECES = Stor<S>::PIECES;
    static constexpr int ELEMS_PER_PIECE = 16 / sizeof(S);
    static constexpr int TOTAL = 3 * ROWS * PIECES;
};

// Issue the global loads of chunk c. The loads are unconditional (addresses are
// clamped into the sequence) so no branch separates a load from its use; rows
// past the end of the sequence are zeroed when the tile is written to LDS.
template <typename S, int PPT>
__device__ __forceinline__ void load_chunk(uint4 (&pf)[PPT], float& pe, int c, int b, int N, int tid,
                                           const S* Qu, const S* Ku, const S* Vu,
                                           const float* etau, float eta_const)
{
    using P = Pieces<S>;
    const int c0 = c * b;
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int idx = min(tid + k * THREADS, P::TOTAL - 1);
        const int tensor = idx / (ROWS * P::PIECES);
        const int rem = idx - tensor * (ROWS * P::PIECES);
        const int row = rem / P::PIECES;
        const int piece = rem - row * P::PIECES;
        const S* src = tensor == 0 ? Qu : (tensor == 1 ? Ku : Vu);
        const int srow = min(c0 + row, N - 1);
        pf[k] = *reinterpret_cast<const uint4*>(src + (size_t)srow * D + piece * P::ELEMS_PER_PIECE);
    }
    pe = etau ? etau[min(c0 + (tid & (ROWS - 1)), N - 1)] : eta_const;
}

// Write a prefetched chunk of bc valid rows into an LDS stage (other rows zero).
template <typename S, int PPT>
__device__ __forceinline__ void store_chunk(Stage<S>& st, const uint4 (&pf)[PPT], float pe, int tid,
                                            int bc)
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
            const bool keep = row < bc;
            uint4 v;
            v.x = keep ? pf[k].x : 0u;
            v.y = keep ? pf[k].y : 0u;
            v.z = keep ? pf[k].z : 0u;
            v.w = keep ? pf[k].w : 0u;
            *reinterpret_cast<uint4*>(dst + row * Stor<S>::STRIDE + piece * P::ELEMS_PER_PIECE) = v;
        }
    }
    if (tid < ROWS) st.eta[tid] = tid < bc ? pe : 0.f;
}


}  // namespace smallb
}  // namespace ttt

namespace ttt {
namespace smallb {

// Row sums over the 64 columns of a 16-row block held in the C layout by the
// four waves (wave w holds columns 16w..16w+15): a[i], b[i] are this lane's
// values for rows 4g+i on entry and the full row totals on return. Contains one
// workgroup barrier; `red` is a [4][ROWS][2] LDS exchange buffer that must not be
// rewritten before every wave has passed the next barrier.
__device__ __forceinline__ void xwave_row_sums(float (&a)[4], float (&b)[4], float (*red)[ROWS][2],
                                               int w, int g, int n)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = row16_sum(a[i]);
        b[i] = row16_sum(b[i]);
    }
    if (n == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            red[w][4 * g + i][0] = a[i];
            red[w][4 * g + i][1] = b[i];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float x = 0.f, y = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            x += red[ww][4 * g + i][0];
            y += red[ww][4 * g + i][1];
        }
        a[i] = x;
        b[i] = y;
    }
}

// B operand of a 16x16x32 product from two C-layout accumulator tiles holding
// rows [32p, 32p+16) and [32p+16, 32p+32) of a state matrix (permuted k order:
// slot j < 4 is row 4g+j of the first tile, slot j >= 4 row 4g+j-4 of the second).
template <int T>
__device__ __forceinline__ void b8_from_acc(const f32x4& t0, const f32x4& t1, bf16x8 (&out)[T])
{
    const float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
    terms8<T>(x, out);
}

}  // namespace smallb
}  // namespace ttt

namespace ttt {
namespace smallb {


// A operand (16x16x16) of K^T for feature tile r: lane (g, n) gets
// K[4g + j][16r + n], j = 0..3, i.e. four consecutive tokens of one feature.
// bf16 tiles use the LDS transpose read: lane (g, n) addresses row 4g + n/4,
// elements 16r + 4(n%4) .. +3, and the hardware hands back the column.
template <typename S, int T>
__device__ __forceinline__ void load_kT_tile(const S* k, int r, int g, int n, bf16x4 (&out)[T])
{
    if constexpr (sizeof(S) == 2) {
        static_assert(T == 1, "bf16 streams are exact in one term");
        typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
        const S* p = k + (4 * g + (n >> 2)) * Stor<S>::STRIDE + 16 * r + 4 * (n & 3);
        out[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(p));
    } else {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = k[(4 * g + j) * Stor<S>::STRIDE + 16 * r + n];
        terms4<T>(x, out);
    }
}

// Four consecutive elements p[0..3] as fp32.
template <typename S>
__device__ __forceinline__ float4 load4_f32(const S* p)
{
    if constexpr (sizeof(S) == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        return make_float4(__builtin_bit_cast(float, v.x << 16), __builtin_bit_cast(float, v.x & 0xFFFF0000u),
                           __builtin_bit_cast(float, v.y << 16), __builtin_bit_cast(float, v.y & 0xFFFF0000u));
    } else {
        return *reinterpret_cast<const float4*>(p);
    }
}

}  // namespace smallb
}  // namespace ttt
