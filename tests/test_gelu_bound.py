"""The GELU of the TTT-MLP kernel takes erf from Abramowitz & Stegun, "Handbook
of Mathematical Functions", formula 7.1.26, whose stated absolute error bound
is 1.5e-7. This pins the formula as the kernel writes it (its coefficients, the
odd extension, Phi = (1 + erf) / 2 and the derivative's shared Gaussian factor)
against the exact erf on a dense grid, evaluated in fp32 as on the GPU."""
import math

import numpy as np

P, A1, A2, A3, A4, A5 = 0.3275911, 0.254829592, -0.284496736, 1.421413741, -1.453152027, 1.061405429


def as_phi(a):
    f = np.float32
    a = a.astype(f)
    x = np.abs(a) * f(0.70710678118654752)
    t = f(1) / (f(P) * x + f(1))
    gauss = np.exp(-x * x).astype(f)
    poly = t * (f(A1) + t * (f(A2) + t * (f(A3) + t * (f(A4) + t * f(A5)))))
    erfx = f(1) - poly * gauss
    return f(0.5) * (f(1) + np.copysign(erfx, a)), gauss


def test_phi_and_gelu_within_the_published_bound():
    a = np.linspace(-12.0, 12.0, 200001)
    phi, gauss = as_phi(a)
    exact_phi = np.array([0.5 * (1.0 + math.erf(v / math.sqrt(2.0))) for v in a])
    # 1.5e-7 / 2 from the formula, plus the fp32 evaluation: 1 - poly exp(-x^2)
    # cancels to a small erf near x = 0 where poly exp(-x^2) is close to 1, so a
    # few 2^-24 roundings of order-one terms add up to ~2e-7 there
    assert np.max(np.abs(phi - exact_phi)) < 4e-7
    gelu_d = phi + a * 0.39894228040143267794 * gauss
    exact_d = exact_phi + a * np.exp(-0.5 * a * a) / math.sqrt(2.0 * math.pi)
    assert np.max(np.abs(gelu_d - exact_d)) < 6e-7
