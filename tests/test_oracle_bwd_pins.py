"""Pins of the oracle's backward of TTT-Linear (``oracle.linear_bwd``): its
gradients are checked against central finite differences of the forward oracle
(itself pinned in test_oracle_pins.py), against closed forms, and for
linearity in the upstream gradients.

The objective is L = sum(dZ * Z) + sum(dW_end * W_end) with fixed random dZ,
dW_end, so dL/dX is exactly what linear_bwd returns for every input X.
"""
import numpy as np
import pytest

import oracle

EPS = 1e-6


def problem(rng, kind, B=2, H=2, N=11, d=5, b=4):
    Q = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    K = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    V = rng.standard_normal((B, H, N, d))
    eta = rng.uniform(0.05, 0.4, (B, H, N))
    W0 = rng.standard_normal((B, H, d, d)) / np.sqrt(d)
    gamma = 1.0 + 0.3 * rng.standard_normal((H, d)) if kind == oracle.LN else None
    beta = 0.3 * rng.standard_normal((H, d)) if kind == oracle.LN else None
    dZ = rng.standard_normal((B, H, N, d))
    dWe = rng.standard_normal((B, H, d, d))
    return dict(Q=Q, K=K, V=V, eta=eta, W0=W0, gamma=gamma, beta=beta), dZ, dWe, b


def objective(kind, x, b, dZ, dWe):
    Z, We = oracle.linear(oracle.DUAL, kind, x["Q"], x["K"], x["V"], x["eta"], x["W0"], b, x["gamma"],
                          x["beta"], EPS)
    return float(np.sum(dZ * Z) + np.sum(dWe * We))


def analytic(kind, x, b, dZ, dWe):
    return oracle.linear_bwd(kind, x["Q"], x["K"], x["V"], x["eta"], x["W0"], b, dZ, dWe, x["gamma"],
                             x["beta"], EPS)


GRAD = {"Q": "dQ", "K": "dK", "V": "dV", "eta": "deta", "W0": "dW0", "gamma": "dgamma", "beta": "dbeta"}


@pytest.mark.parametrize("kind", [oracle.PLAIN, oracle.LN])
@pytest.mark.parametrize("b", [1, 4, 16])
def test_gradients_match_finite_differences(kind, b):
    """Central differences (step 1e-5) of the forward oracle at 10 random entries
    of every input, including a ragged last chunk (N = 11) and per-token eta."""
    rng = np.random.default_rng(100 + 10 * kind + b)
    x, dZ, dWe, _ = problem(rng, kind, b=b)
    g = analytic(kind, x, b, dZ, dWe)
    h = 1e-5
    for name, gname in GRAD.items():
        if x[name] is None:
            assert g[gname] is None
            continue
        arr = x[name]
        flat = arr.reshape(-1)
        for idx in rng.choice(flat.size, size=min(10, flat.size), replace=False):
            saved = flat[idx]
            flat[idx] = saved + h
            lp = objective(kind, x, b, dZ, dWe)
            flat[idx] = saved - h
            lm = objective(kind, x, b, dZ, dWe)
            flat[idx] = saved
            fd = (lp - lm) / (2 * h)
            an = g[gname].reshape(-1)[idx]
            assert abs(fd - an) <= 1e-7 * (1.0 + abs(fd)), (name, idx, fd, an)


def test_zero_step_closed_form():
    """eta = 0 (plain): the state never moves, Z = Q W0 and W_end = W0, so
    dQ = dZ W0^T, dK = dV = 0 and dW0 = sum_t q_t^T dz_t + dW_end."""
    rng = np.random.default_rng(7)
    x, dZ, dWe, b = problem(rng, oracle.PLAIN)
    x["eta"] = np.zeros_like(x["eta"])
    g = analytic(oracle.PLAIN, x, b, dZ, dWe)
    assert np.allclose(g["dQ"], dZ @ np.swapaxes(x["W0"], -1, -2), atol=1e-13)
    assert np.all(g["dK"] == 0) and np.all(g["dV"] == 0)
    dW0 = np.swapaxes(x["Q"], -1, -2) @ dZ + dWe
    assert np.allclose(g["dW0"], dW0, atol=1e-12)


def test_plain_one_token_closed_form():
    """One token, plain f, eta scalar: W1 = W0 - 2 eta k^T (k W0 - v), z = q W1.
    With dZ only: dv = 2 eta (q k^T) dz, written out by hand."""
    rng = np.random.default_rng(8)
    d = 4
    q, k, v = rng.standard_normal((3, d))
    W0 = rng.standard_normal((d, d))
    eta = 0.3
    dz = rng.standard_normal(d)
    g = oracle.linear_bwd(oracle.PLAIN, q.reshape(1, 1, 1, d), k.reshape(1, 1, 1, d), v.reshape(1, 1, 1, d),
                          eta, W0.reshape(1, 1, d, d), 1, dz.reshape(1, 1, 1, d))
    # z = q W0 - 2 eta (q.k) (k W0 - v): dz/dv = 2 eta (q.k) I
    assert np.allclose(g["dV"].reshape(d), 2 * eta * np.dot(q, k) * dz, atol=1e-14)
    # d/d eta = -2 (q.k) (k W0 - v) . dz
    assert np.isclose(g["deta"].reshape(()), -2 * np.dot(q, k) * np.dot(k @ W0 - v, dz), atol=1e-14)


@pytest.mark.parametrize("kind", [oracle.PLAIN, oracle.LN])
def test_linear_in_upstream_gradients(kind):
    rng = np.random.default_rng(9 + kind)
    x, dZ, dWe, b = problem(rng, kind)
    ga = analytic(kind, x, b, dZ, None)
    gb = analytic(kind, x, b, np.zeros_like(dZ), dWe)
    gc = analytic(kind, x, b, dZ, dWe)
    for k in GRAD.values():
        if gc[k] is None:
            continue
        assert np.allclose(gc[k], ga[k] + gb[k], atol=1e-12)
