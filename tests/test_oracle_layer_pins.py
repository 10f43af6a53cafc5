"""Pins of the oracle's whole-layer function (projections, key normalisation,
output LayerNorm + residual + output projection) against facts that the pages
and the mathematics fix.

Page 1 is "Test-Time Training: Linear Complexity Beyond Attention": section
"1. The Self-Supervised Inner-Loop Task" defines the projections, section
"3. Forward Evaluation and Output Projection" the output, and the page's layer
code normalises keys. The inner model itself is pinned in test_oracle_pins.py.
"""
import numpy as np
import pytest


def rel(a, b):
    den = np.max(np.abs(b))
    num = np.max(np.abs(a - b))
    return num if den == 0 else num / den


def problem(rng, B=2, N=24, H=2, d=8, D=None, kind=1):
    D = D or H * d
    HD = H * d
    x = rng.standard_normal((B, N, D))
    Wq = rng.standard_normal((HD, D)) / np.sqrt(D)
    Wk = rng.standard_normal((HD, D)) / np.sqrt(D)
    Wv = rng.standard_normal((HD, D)) / np.sqrt(D)
    Wo = rng.standard_normal((D, HD)) / np.sqrt(HD)
    eta = rng.uniform(0.05, 0.3, (B, H, N))
    W0 = rng.standard_normal((B, H, d, d)) / np.sqrt(d)
    g = 1.0 + 0.3 * rng.standard_normal((H, d))
    bt = 0.3 * rng.standard_normal((H, d))
    go = 1.0 + 0.3 * rng.standard_normal((H, d))
    bo = 0.3 * rng.standard_normal((H, d))
    return dict(kind=kind, x=x, Wq=Wq, Wk=Wk, Wv=Wv, Wo=Wo, eta=eta, W0=W0, b=4, H=H,
                gamma=g, beta=bt, gamma_o=go, beta_o=bo)


def run(oracle_mod, p, **over):
    q = dict(p)
    q.update(over)
    return oracle_mod.layer(**q)


def test_projection_orientation_and_head_split(oracle_mod):
    """Section 1: q_t = W_Q x_t with W_Q of shape [H*d, D]. With W_Q a
    permutation matrix (W_Q[o, perm[o]] = 1) query entry o is x entry perm[o],
    and head h holds outputs h*d .. h*d+d-1. A transposed W_Q would select
    perm^-1 instead, a wrong head split would move entries between heads."""
    rng = np.random.default_rng(11)
    p = problem(rng, H=3, d=4, D=12)
    perm = rng.permutation(12)
    assert np.any(perm[perm] != np.arange(12))       # not an involution
    P = np.zeros((12, 12))
    P[np.arange(12), perm] = 1.0
    perm_v = rng.permutation(12)
    Pv = np.zeros((12, 12))
    Pv[np.arange(12), perm_v] = 1.0
    _, _, parts = run(oracle_mod, p, Wq=P, Wv=Pv)
    x = p["x"]
    for h in range(3):
        for j in range(4):
            assert np.array_equal(parts["Q"][:, h, :, j], x[:, :, perm[4 * h + j]])
            assert np.array_equal(parts["V"][:, h, :, j], x[:, :, perm_v[4 * h + j]])


def test_keys_have_unit_length_and_scale_out(oracle_mod):
    """The page's layer code normalises each key to unit L2 length, so every
    key row has norm 1 and scaling W_K by any positive factor changes nothing."""
    rng = np.random.default_rng(12)
    p = problem(rng)
    y, We, parts = run(oracle_mod, p)
    nrm = np.sqrt(np.sum(parts["K"] ** 2, axis=-1))
    assert np.max(np.abs(nrm - 1.0)) < 1e-13
    y2, We2, _ = run(oracle_mod, p, Wk=3.7 * p["Wk"])
    assert rel(y2, y) < 1e-12 and rel(We2, We) < 1e-12
    # ... while scaling W_V does change the output (the normalisation is on k only)
    y3, _, _ = run(oracle_mod, p, Wv=3.7 * p["Wv"])
    assert rel(y3, y) > 1e-3


def test_zero_key_stays_zero(oracle_mod):
    """A token whose key is zero contributes nothing to the inner update
    (k = 0 makes k^T g = 0) and produces no NaN."""
    rng = np.random.default_rng(13)
    p = problem(rng)
    x = p["x"].copy()
    x[0, 5, :] = 0.0
    y, We, parts = run(oracle_mod, p, x=x)
    assert np.all(np.isfinite(y))
    assert np.all(parts["K"][0, :, 5, :] == 0.0)


def test_output_layernorm_closed_form(oracle_mod):
    """Section 3 with W_O = I, gamma_o = 1, beta_o = 0: y - q is LayerNorm(z),
    which has mean 0 and mean square var / (var + eps) over each head."""
    rng = np.random.default_rng(14)
    H, d = 2, 8
    p = problem(rng, H=H, d=d)
    eps = 1e-12
    y, _, parts = run(oracle_mod, p, Wo=np.eye(H * d), gamma_o=np.ones((H, d)),
                      beta_o=np.zeros((H, d)), eps=eps)
    B, N = p["x"].shape[:2]
    qrow = parts["Q"].transpose(0, 2, 1, 3).reshape(B, N, H * d)
    a = (y - qrow).reshape(B, N, H, d)
    assert np.max(np.abs(a.mean(axis=-1))) < 1e-12
    assert np.max(np.abs((a * a).mean(axis=-1) - 1.0)) < 1e-9


def test_zero_state_zero_step_closed_form(oracle_mod):
    """W0 = 0 and eta = 0 (TTT-Linear, plain f): the state never moves, so
    z = f(q; 0) = 0, LayerNorm(0) = beta_o, and y = W_O (W_Q x + beta_o), here
    evaluated as x (W_O W_Q)^T + W_O beta_o."""
    rng = np.random.default_rng(15)
    p = problem(rng, H=2, d=8, D=24, kind=0)
    B, N = p["x"].shape[:2]
    W0 = np.zeros_like(p["W0"])
    y, We, _ = run(oracle_mod, p, W0=W0, eta=0.0)
    expect = p["x"] @ (p["Wo"] @ p["Wq"]).T + p["Wo"] @ p["beta_o"].reshape(-1)
    assert rel(y, expect) < 1e-13
    assert np.all(We == 0.0)


def test_linear_in_output_projection(oracle_mod):
    """y is linear in W_O."""
    rng = np.random.default_rng(16)
    p = problem(rng, D=20)
    Wo2 = rng.standard_normal(p["Wo"].shape)
    ya, _, _ = run(oracle_mod, p)
    yb, _, _ = run(oracle_mod, p, Wo=Wo2)
    yc, _, _ = run(oracle_mod, p, Wo=p["Wo"] + Wo2)
    assert rel(yc, ya + yb) < 1e-12


@pytest.mark.parametrize("kind", [0, 1])
def test_causal_and_sequences_independent(oracle_mod, kind):
    """Outputs at tokens before t0 do not depend on token t0 (the inner loop
    only looks back), and each sequence of the batch is processed alone."""
    rng = np.random.default_rng(17 + kind)
    p = problem(rng, N=23, kind=kind)
    y, We, _ = run(oracle_mod, p)
    x = p["x"].copy()
    t0 = 10                                   # inside the third chunk of 4
    x[0, t0, :] += 1.0
    y2, _, _ = run(oracle_mod, p, x=x)
    assert rel(y2[0, :t0], y[0, :t0]) < 1e-13
    assert rel(y2[0, t0], y[0, t0]) > 1e-6
    assert np.array_equal(y2[1], y[1])
    one = dict(p, x=p["x"][1:], eta=p["eta"][1:], W0=p["W0"][1:])
    y1, We1, _ = oracle_mod.layer(**one)
    assert rel(y1[0], y[1]) < 1e-13 and rel(We1[0], We[1]) < 1e-13
