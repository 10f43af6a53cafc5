// decode.hip -- single-token decode step of TTT-Linear (plain or LayerNorm +
// residual inner model), d = 64, for B*H independent (sequence, head) streams.
//
// One token per stream: the online rule of page "Test-Time Training: Linear
// Complexity Beyond Attention" (section "2. The Online Gradient Descent Update
// Rule", output as in section "3. Forward Evaluation and Output Projection"):
//     g   = d ||f(k; W) - v||^2 / d(k W)          (row vector, includes the 2)
//     W  <- W - eta k^T g
//     z   = f(q; W)                               (the updated weights)
// This is the generation-time counterpart of the chunked forward: a mini-batch
// of one token. The state is read and written once per token, so the step is
// bound by moving W (2 * 16 KB per stream).
//
// One wave per stream; lane n owns column n of W (64 fp32 registers). The
// vectors k and q are broadcast through LDS; LayerNorm row statistics are
// reductions over the 64 lanes (DPP within rows of 16, then across rows).
#include "device_common.h"
#include "kernels.h"

namespace ttt {
namespace {

constexpr int DD = 64;

template <typename S>
__device__ __forceinline__ float load_elem(const S* p);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p)
{
    return __builtin_bit_cast(float, (uint32_t)*p << 16);
}

// Sum over the 64 lanes of the wave; every lane gets the result.
__device__ __forceinline__ float wave_sum(float x)
{
    x = row16_sum(x);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
}

// LayerNorm of the 64-lane row h (one entry per lane): returns xhat, sets r.
__device__ __forceinline__ float ln_xhat(float h, float eps, float& r)
{
    const float mu = wave_sum(h) * (1.f / DD);
    const float xc = h - mu;
    const float var = wave_sum(xc * xc) * (1.f / DD);
    r = 1.f / sqrtf(var + eps);
    return xc * r;
}

template <int KIND, typename S>
__global__ void __launch_bounds__(DD)
decode_kernel(int H, const S* __restrict__ q, const S* __restrict__ k, const S* __restrict__ v,
              const float* __restrict__ eta, float eta_const, float* __restrict__ W,
              const float* __restrict__ gamma, const float* __restrict__ beta, float eps, float* __restrict__ z)
{
    __shared__ float kq[2][DD];
    const int unit = blockIdx.x, n = threadIdx.x;
    const size_t vo = (size_t)unit * DD;
    const float kn = load_elem(k + vo + n), qn = load_elem(q + vo + n), vn = load_elem(v + vo + n);
    kq[0][n] = kn;
    kq[1][n] = qn;
    float* Wu = W + (size_t)unit * DD * DD;
    float wc[DD];
#pragma unroll
    for (int i = 0; i < DD; ++i) wc[i] = Wu[i * DD + n];
    __syncthreads();

    // h_n = sum_i k_i W[i][n]
    float hk = 0.f;
#pragma unroll
    for (int i = 0; i < DD; i += 4) {
        const float4 k4 = *reinterpret_cast<const float4*>(&kq[0][i]);
        hk = fmaf(k4.x, wc[i], hk);
        hk = fmaf(k4.y, wc[i + 1], hk);
        hk = fmaf(k4.z, wc[i + 2], hk);
        hk = fmaf(k4.w, wc[i + 3], hk);
    }

    float g, gm = 0.f, bt = 0.f;
    if constexpr (KIND == 0) {
        g = 2.f * (hk - vn);
    } else {
        const int head = unit % H;
        gm = gamma[head * DD + n];
        bt = beta[head * DD + n];
        float r;
        const float xh = ln_xhat(hk, eps, r);
        const float dy = 2.f * ((kn + (gm * xh + bt)) - vn);
        const float dxh = dy * gm;
        const float m1 = wave_sum(dxh) * (1.f / DD);
        const float m2 = wave_sum(dxh * xh) * (1.f / DD);
        g = r * ((dxh - m1) - xh * m2);
    }

    // W[:, n] -= eta k^T g_n
    const float step = (eta ? eta[unit] : eta_const) * g;
#pragma unroll
    for (int i = 0; i < DD; i += 4) {
        const float4 k4 = *reinterpret_cast<const float4*>(&kq[0][i]);
        wc[i] = fmaf(-step, k4.x, wc[i]);
        wc[i + 1] = fmaf(-step, k4.y, wc[i + 1]);
        wc[i + 2] = fmaf(-step, k4.z, wc[i + 2]);
        wc[i + 3] = fmaf(-step, k4.w, wc[i + 3]);
    }

    // z = f(q; W) with the updated weights
    float hq = 0.f;
#pragma unroll
    for (int i = 0; i < DD; i += 4) {
        const float4 q4 = *reinterpret_cast<const float4*>(&kq[1][i]);
        hq = fmaf(q4.x, wc[i], hq);
        hq = fmaf(q4.y, wc[i + 1], hq);
        hq = fmaf(q4.z, wc[i + 2], hq);
        hq = fmaf(q4.w, wc[i + 3], hq);
    }
    float out = hq;
    if constexpr (KIND == 1) {
        float r;
        const float xh = ln_xhat(hq, eps, r);
        out = qn + (gm * xh + bt);
    }
#pragma unroll
    for (int i = 0; i < DD; ++i) Wu[i * DD + n] = wc[i];
    z[vo + n] = out;
}

}  // namespace

hipError_t launch_decode_linear(const LinearArgs& a, hipStream_t stream)
{
    const int units = a.B * a.H;
    if (a.kind == 0 && a.dtype == 0)
        hipLaunchKernelGGL((decode_kernel<0, float>), dim3(units), dim3(DD), 0, stream, a.H,
                           static_cast<const float*>(a.Q), static_cast<const float*>(a.K),
                           static_cast<const float*>(a.V), a.eta, a.eta_const, a.W_end, a.gamma, a.beta, a.eps, a.Z);
    else if (a.kind == 0)
        hipLaunchKernelGGL((decode_kernel<0, uint16_t>), dim3(units), dim3(DD), 0, stream, a.H,
                           static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                           static_cast<const uint16_t*>(a.V), a.eta, a.eta_const, a.W_end, a.gamma, a.beta, a.eps,
                           a.Z);
    else if (a.dtype == 0)
        hipLaunchKernelGGL((decode_kernel<1, float>), dim3(units), dim3(DD), 0, stream, a.H,
                           static_cast<const float*>(a.Q), static_cast<const float*>(a.K),
                           static_cast<const float*>(a.V), a.eta, a.eta_const, a.W_end, a.gamma, a.beta, a.eps, a.Z);
    else
        hipLaunchKernelGGL((decode_kernel<1, uint16_t>), dim3(units), dim3(DD), 0, stream, a.H,
                           static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                           static_cast<const uint16_t*>(a.V), a.eta, a.eta_const, a.W_end, a.gamma, a.beta, a.eps,
                           a.Z);
    return hipGetLastError();
}

}  // namespace ttt
