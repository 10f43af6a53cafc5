// device_common.h -- gfx950 device helpers shared by the TTT kernels:
// MFMA operand vector types and wrappers, fp32 -> bf16 multi-term splitting,
// DPP row reductions.
//
// MFMA register layouts used throughout (checked on gfx950 hardware):
//   v_mfma_f32_16x16x32_bf16  A[16x32]: lane l holds row l%16, k = 8*(l/16) + j (j<8)
//                             B[32x16]: lane l holds col l%16, k = 8*(l/16) + j
//   v_mfma_f32_16x16x16_bf16  A[16x16]: lane l holds row l%16, k = 4*(l/16) + j (j<4)
//                             B[16x16]: lane l holds col l%16, k = 4*(l/16) + j
//   both                      C[16x16]: lane l holds col l%16, rows 4*(l/16) + i (i<4)
//   v_mfma_f32_32x32x16_bf16  A[32x16]: lane l holds row l%32, k = 8*(l/32) + j
//                             B[16x32]: lane l holds col l%32, k = 8*(l/32) + j
//                             C[32x32]: lane l holds col l%32,
//                                       rows 8*(i/4) + 4*(l/32) + i%4 (i<16)
// A C-layout 16x16 tile therefore IS a valid B operand of a 16x16x16 product
// (k index = C row), and, up to a fixed permutation of k, of a 16x16x32 one.
//
// Precision scheme: an fp32 operand x is carried as T bf16 terms
// x ~ t0 + t1 + ... (t0 = bf16(x), t1 = bf16(x - t0), ...), and a product of a
// T_a-term and a T_b-term operand keeps the term pairs (i, j) with
// i + j < max(T_a, T_b). Two terms carry 16 significant bits, three carry 24
// (fp32). bf16 token streams are exact in one term.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4;  // 16x16x16 operand
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x16(const bf16x4& a, const bf16x4& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ short bf16_bits(__bf16 x) { return __builtin_bit_cast(short, x); }
__device__ __forceinline__ __bf16 bits_bf16(uint16_t x) { return __builtin_bit_cast(__bf16, x); }
__device__ __forceinline__ float bf16_to_f32(__bf16 x) { return (float)x; }

// Split fp32 x into T bf16 terms (round to nearest even at each step).
template <int T>
__device__ __forceinline__ void split_terms(float x, __bf16 (&t)[T])
{
#pragma unroll
    for (int i = 0; i < T; ++i) {
        t[i] = (__bf16)x;
        x -= (float)t[i];
    }
}

// acc += sum over kept term pairs of A_i * B_j (16x16x32 shape).
template <int TA, int TB>
__device__ __forceinline__ f32x4 mma32_terms(f32x4 acc, const bf16x8 (&a)[TA], const bf16x8 (&b)[TB])
{
    constexpr int T = TA > TB ? TA : TB;
#pragma unroll
    for (int s = T - 1; s >= 0; --s) {        // smallest contributions first
#pragma unroll
        for (int i = 0; i < TA; ++i) {
            const int j = s - i;
            if (j >= 0 && j < TB) acc = mfma_16x16x32(a[i], b[j], acc);
        }
    }
    return acc;
}

// acc += sum over kept term pairs of A_i * B_j (16x16x16 shape).
template <int TA, int TB>
__device__ __forceinline__ f32x4 mma16_terms(f32x4 acc, const bf16x4 (&a)[TA], const bf16x4 (&b)[TB])
{
    constexpr int T = TA > TB ? TA : TB;
#pragma unroll
    for (int s = T - 1; s >= 0; --s) {
#pragma unroll
        for (int i = 0; i < TA; ++i) {
            const int j = s - i;
            if (j >= 0 && j < TB) acc = mfma_16x16x16(a[i], b[j], acc);
        }
    }
    return acc;
}

// ---------------------------------------------------------------------------
// DPP cross-lane moves inside a row of 16 lanes
// ---------------------------------------------------------------------------
enum : int {
    DPP_QUAD_XOR1 = 0xB1,       // quad_perm [1,0,3,2]
    DPP_QUAD_XOR2 = 0x4E,       // quad_perm [2,3,0,1]
    DPP_ROW_HALF_MIRROR = 0x141,
    DPP_ROW_MIRROR = 0x140,
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the result.
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp_mov<DPP_QUAD_XOR1>(x);
    x += dpp_mov<DPP_QUAD_XOR2>(x);
    x += dpp_mov<DPP_ROW_HALF_MIRROR>(x);
    x += dpp_mov<DPP_ROW_MIRROR>(x);
    return x;
}

}  // namespace ttt
