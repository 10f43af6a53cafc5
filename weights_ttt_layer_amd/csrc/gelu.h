// gelu.h -- GELU in its erf form for the TTT-MLP kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace ttt {

// GELU(a) = a Phi(a), Phi(a) = (1 + erf(a / sqrt 2)) / 2, and its derivative
// Phi(a) + a phi(a). erf comes from Abramowitz & Stegun, "Handbook of
// Mathematical Functions", formula 7.1.26: for x >= 0,
//     erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
//     t = 1 / (1 + p x),   |error| <= 1.5e-7,
// extended to x < 0 by odd symmetry. Only Phi = (1 + erf) / 2 is used, so the
// absolute error bound is the one that matters. exp(-x^2) = exp(-a^2 / 2) is
// also the Gaussian factor of phi, shared by the derivative.
constexpr float AS_P = 0.3275911f;
constexpr float AS_A1 = 0.254829592f, AS_A2 = -0.284496736f, AS_A3 = 1.421413741f,
                AS_A4 = -1.453152027f, AS_A5 = 1.061405429f;

__device__ __forceinline__ float phi_cdf(float a, float& gauss)
{
    const float x = fabsf(a) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(AS_P, x, 1.f));
    gauss = __expf(-x * x);
    const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, AS_A5, AS_A4), AS_A3), AS_A2), AS_A1);
    const float erfx = 1.f - poly * gauss;
    return 0.5f * (1.f + copysignf(erfx, a));
}

__device__ __forceinline__ float gelu_f(float a)
{
    float gauss;
    return a * phi_cdf(a, gauss);
}

// GELU(a) and d/da GELU(a) = Phi(a) + a exp(-a^2/2) / sqrt(2 pi)
__device__ __forceinline__ void gelu_fd(float a, float& f, float& fd)
{
    float gauss;
    const float c = phi_cdf(a, gauss);
    f = a * c;
    fd = fmaf(a * 0.39894228040143267794f, gauss, c);
}

}  // namespace ttt
