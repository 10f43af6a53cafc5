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

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma_32x32x16_f16(const f16x8& a, const f16x8& b, const f32x16& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Logical index of workgroup x of `total`. Workgroups are dealt to the eight
// XCDs round robin (workgroup x runs on XCD x % 8); this gives XCD c a
// contiguous range of logical indices, so neighbours in logical order share
// that XCD's L2.
__device__ __forceinline__ int xcd_tile(int x, int total)
{
    const int per = total >> 3, rem = total & 7, c = x & 7, k = x >> 3;
    return c < rem ? c * (per + 1) + k : rem * (per + 1) + (c - rem) * per + k;
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

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 and packed into one register (element 0 in
// the low half): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Two fp32 values rounded to fp16 (nearest even) and packed into one register.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b)
{
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// Split the pair (a, b) into T packed bf16 pairs: out[0] = bf16(a, b),
// out[1] = bf16 of the remainders, ...
template <int T>
__device__ __forceinline__ void split_pair(float a, float b, uint32_t (&out)[T])
{
#pragma unroll
    for (int i = 0; i < T; ++i) {
        out[i] = pack_bf16x2(a, b);
        if (i + 1 < T) {
            a -= __builtin_bit_cast(float, out[i] << 16);
            b -= __builtin_bit_cast(float, out[i] & 0xFFFF0000u);
        }
    }
}

// Eight fp32 values as T bf16x8 operand terms.
template <int T>
__device__ __forceinline__ void terms8(const float (&x)[8], bf16x8 (&out)[T])
{
    uint32_t p[4][T];
#pragma unroll
    for (int q = 0; q < 4; ++q) split_pair<T>(x[2 * q], x[2 * q + 1], p[q]);
#pragma unroll
    for (int s = 0; s < T; ++s) out[s] = __builtin_bit_cast(bf16x8, make_uint4(p[0][s], p[1][s], p[2][s], p[3][s]));
}

// Four fp32 values as T bf16x4 (16x16x16) operand terms.
template <int T>
__device__ __forceinline__ void terms4(const float (&x)[4], bf16x4 (&out)[T])
{
    uint32_t p[2][T];
    split_pair<T>(x[0], x[1], p[0]);
    split_pair<T>(x[2], x[3], p[1]);
#pragma unroll
    for (int s = 0; s < T; ++s) out[s] = __builtin_bit_cast(bf16x4, make_uint2(p[0][s], p[1][s]));
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

// Sum over the four 16-lane rows of a wave (lanes n, n+16, n+32, n+48); every
// lane gets the total. v_permlane32_swap / v_permlane16_swap pair each lane with
// its xor-32 / xor-16 partner.
__device__ __forceinline__ float xrow4_sum(float x)
{
    const int xi = __builtin_bit_cast(int, x);
    auto a = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    x = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
    const int yi = __builtin_bit_cast(int, x);
    auto b = __builtin_amdgcn_permlane16_swap(yi, yi, false, false);
    return __builtin_bit_cast(float, (int)b[0]) + __builtin_bit_cast(float, (int)b[1]);
}

// Both sums of xrow4_sum for two values at once, in the same order of
// additions. v_permlane32_swap of (a, b) leaves rows 0-1 of a and b in the
// first result and rows 2-3 in the second, so their sum holds a's half-sums in
// lanes 0-31 and b's in lanes 32-63; v_permlane16_swap then completes both, and
// a last v_permlane32_swap hands every lane both totals.
__device__ __forceinline__ void xrow4_sum2(float& a, float& b)
{
    auto s1 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, a), __builtin_bit_cast(int, b), false, false);
    const float y = __builtin_bit_cast(float, (int)s1[0]) + __builtin_bit_cast(float, (int)s1[1]);
    const int yi = __builtin_bit_cast(int, y);
    auto s2 = __builtin_amdgcn_permlane16_swap(yi, yi, false, false);
    const float z = __builtin_bit_cast(float, (int)s2[0]) + __builtin_bit_cast(float, (int)s2[1]);
    const int zi = __builtin_bit_cast(int, z);
    auto s3 = __builtin_amdgcn_permlane32_swap(zi, zi, false, false);
    a = __builtin_bit_cast(float, (int)s3[0]);
    b = __builtin_bit_cast(float, (int)s3[1]);
}

// ---------------------------------------------------------------------------
// Direct global->LDS loads
// ---------------------------------------------------------------------------
// One 16-byte (dma16) or 4-byte (dma4) direct global->LDS load per lane: lane
// l's bytes land at lds + 16 l (+ 4 l). Issued as assembly so that the compiler
// does not track them: it cannot tell LDS buffers apart through the loads'
// addresses and would otherwise wait for a prefetch before every read of
// another buffer. The caller waits for these loads explicitly (vmcnt) before
// the barrier that publishes the data. (M0 written by SALU needs one wait
// state before an LDS-DMA instruction.)
__device__ __forceinline__ void dma16(const void* g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ void dma4(const void* g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

}  // namespace ttt
