// peak.hip -- calibration kernels behind include/ttt_peak.h: a plain copy (the
// HBM bandwidth this device reaches), an MFMA loop (the dense bf16 matrix-core
// rate it reaches) and the device's compute-unit count and clock. Built into
// libttt_peak.so, separate from the layer library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ttt_peak.h"

namespace {

constexpr int PEAK_THREADS = 256;
constexpr int COPY_UNROLL = 4;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// Grid-stride copy of n 16-byte elements; each thread keeps COPY_UNROLL loads in
// flight before its stores.
__global__ void __launch_bounds__(PEAK_THREADS) peak_copy_kernel(const uint4* __restrict__ src,
                                                                  uint4* __restrict__ dst, size_t n)
{
    const size_t stride = (size_t)gridDim.x * PEAK_THREADS;
    for (size_t i = (size_t)blockIdx.x * PEAK_THREADS + threadIdx.x; i < n; i += COPY_UNROLL * stride) {
        uint4 v[COPY_UNROLL];
#pragma unroll
        for (int u = 0; u < COPY_UNROLL; ++u) {
            const size_t j = i + u * stride;
            if (j < n) v[u] = src[j];
        }
#pragma unroll
        for (int u = 0; u < COPY_UNROLL; ++u) {
            const size_t j = i + u * stride;
            if (j < n) dst[j] = v[u];
        }
    }
}

// Four independent accumulation chains per wave, so consecutive MFMAs never
// wait for each other's results.
__global__ void __launch_bounds__(PEAK_THREADS) peak_mfma_kernel(float* __restrict__ out, int iters)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(1e-3f * (float)(lane + j));
        b[j] = (__bf16)(1e-3f * (float)(lane - j));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += (c0[i] + c1[i]) + (c2[i] + c3[i]);
    out[(size_t)blockIdx.x * PEAK_THREADS + threadIdx.x] = s;
}

constexpr int ERR_INVALID = 1, ERR_HIP = 4;

}  // namespace

extern "C" int ttt_peak_device_info(int device, int* compute_units, int* clock_khz, int* wavefront_size)
{
    int v = 0;
    if (compute_units) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return ERR_HIP;
        *compute_units = v;
    }
    if (clock_khz) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeClockRate, device) != hipSuccess) return ERR_HIP;
        *clock_khz = v;
    }
    if (wavefront_size) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeWarpSize, device) != hipSuccess) return ERR_HIP;
        *wavefront_size = v;
    }
    return 0;
}

extern "C" int ttt_peak_copy(const void* src, void* dst, size_t bytes, void* hip_stream)
{
    if (!src || !dst || bytes == 0 || bytes % 16 != 0) return ERR_INVALID;
    if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return ERR_INVALID;
    const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
    if (s < d + bytes && d < s + bytes) return ERR_INVALID;
    const size_t n = bytes / 16;
    size_t blocks = (n + (size_t)PEAK_THREADS * COPY_UNROLL - 1) / ((size_t)PEAK_THREADS * COPY_UNROLL);
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(peak_copy_kernel, dim3((unsigned)blocks), dim3(PEAK_THREADS), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), static_cast<const uint4*>(src),
                       static_cast<uint4*>(dst), n);
    return hipGetLastError() == hipSuccess ? 0 : ERR_HIP;
}

extern "C" int ttt_peak_mfma(float* out, int blocks, int iters, void* hip_stream)
{
    if (!out || blocks < 1 || iters < 1) return ERR_INVALID;
    hipLaunchKernelGGL(peak_mfma_kernel, dim3(blocks), dim3(PEAK_THREADS), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), out, iters);
    return hipGetLastError() == hipSuccess ? 0 : ERR_HIP;
}

extern "C" double ttt_peak_mfma_flops(int blocks, int iters)
{
    return (double)blocks * (PEAK_THREADS / 64) * (double)iters * 4.0 * (2.0 * 32 * 32 * 16);
}
