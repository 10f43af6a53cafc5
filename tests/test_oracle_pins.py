"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test states the passage or the mathematical fact it relies on. Page 1 is
"Test-Time Training: Linear Complexity Beyond Attention"; its sections are
"1. The Self-Supervised Inner-Loop Task", "2. The Online Gradient Descent
Update Rule", "3. Forward Evaluation and Output Projection" and "4. Mini-Batch
Parallelism (Dual Formulation)".
"""
import json
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def rel(a, b):
    """Normwise error max|a-b| / max|b| (0 when both are zero)."""
    den = np.max(np.abs(b))
    num = np.max(np.abs(a - b))
    return num if den == 0 else num / den


def rand_problem(rng, B, H, N, d, hid=None, per_token_eta=True):
    Q = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    K = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    V = rng.standard_normal((B, H, N, d))
    eta = rng.uniform(0.05, 0.4, (B, H, N)) if per_token_eta else 0.2
    gamma = 1.0 + 0.3 * rng.standard_normal((H, d))
    beta = 0.3 * rng.standard_normal((H, d))
    if hid is None:
        W0 = rng.standard_normal((B, H, d, d)) / np.sqrt(d)
        return Q, K, V, eta, W0, gamma, beta
    W1 = rng.standard_normal((B, H, d, hid)) / np.sqrt(d)
    W2 = rng.standard_normal((B, H, hid, d)) / np.sqrt(hid)
    return Q, K, V, eta, W1, W2, gamma, beta


SHAPES = [(2, 2, 5, 4, 3), (1, 2, 64, 8, 16), (2, 1, 37, 8, 4), (1, 1, 7, 4, 16), (1, 1, 9, 4, 1)]


# ---------------------------------------------------------------------------
# P-1: the dual form equals the mini-batch primal form (page 1, section 4:
# the in-batch updates "mirror causal attention" and are an exact rewrite).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,N,d,b", SHAPES)
@pytest.mark.parametrize("kind", [0, 1])
def test_dual_equals_primal_linear(oracle_mod, B, H, N, d, b, kind):
    rng = np.random.default_rng(1 + N * 7 + b + kind)
    Q, K, V, eta, W0, g, bt = rand_problem(rng, B, H, N, d)
    Zp, Wp = oracle_mod.linear(oracle_mod.MINIBATCH, kind, Q, K, V, eta, W0, b, g, bt, 1e-6)
    Zd, Wd = oracle_mod.linear(oracle_mod.DUAL, kind, Q, K, V, eta, W0, b, g, bt, 1e-6)
    assert rel(Zd, Zp) < 1e-12
    assert rel(Wd, Wp) < 1e-12


@pytest.mark.parametrize("B,H,N,d,b", SHAPES)
def test_dual_equals_primal_mlp(oracle_mod, B, H, N, d, b):
    rng = np.random.default_rng(100 + N + b)
    Q, K, V, eta, W1, W2, g, bt = rand_problem(rng, B, H, N, d, hid=4 * d)
    Zp, W1p, W2p = oracle_mod.mlp(oracle_mod.MINIBATCH, Q, K, V, eta, W1, W2, b, g, bt, 1e-6)
    Zd, W1d, W2d = oracle_mod.mlp(oracle_mod.DUAL, Q, K, V, eta, W1, W2, b, g, bt, 1e-6)
    assert rel(Zd, Zp) < 1e-12
    assert rel(W1d, W1p) < 1e-12
    assert rel(W2d, W2p) < 1e-12


def test_dual_differs_from_online_when_b_gt_1(oracle_mod):
    """Guards the pins above against a degenerate oracle: b matters."""
    rng = np.random.default_rng(5)
    Q, K, V, eta, W0, g, bt = rand_problem(rng, 1, 1, 32, 8)
    Z16, _ = oracle_mod.linear(oracle_mod.DUAL, 0, Q, K, V, eta, W0, 16, g, bt)
    Zon, _ = oracle_mod.linear(oracle_mod.ONLINE, 0, Q, K, V, eta, W0, 1, g, bt)
    assert rel(Z16, Zon) > 1e-3


# ---------------------------------------------------------------------------
# P-2: b = 1 reduces to plain online gradient descent (page 1, sections 2-3).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind", [0, 1, "mlp"])
def test_b1_is_online(oracle_mod, kind):
    rng = np.random.default_rng(11)
    if kind == "mlp":
        Q, K, V, eta, W1, W2, g, bt = rand_problem(rng, 2, 2, 23, 4, hid=16)
        ref = oracle_mod.mlp(oracle_mod.ONLINE, Q, K, V, eta, W1, W2, 1, g, bt)
        for mode in (oracle_mod.MINIBATCH, oracle_mod.DUAL):
            got = oracle_mod.mlp(mode, Q, K, V, eta, W1, W2, 1, g, bt)
            for a, r in zip(got, ref):
                assert rel(a, r) < 1e-13
        return
    Q, K, V, eta, W0, g, bt = rand_problem(rng, 2, 2, 23, 8)
    Zo, Wo = oracle_mod.linear(oracle_mod.ONLINE, kind, Q, K, V, eta, W0, 1, g, bt)
    for mode in (oracle_mod.MINIBATCH, oracle_mod.DUAL):
        Z, W = oracle_mod.linear(mode, kind, Q, K, V, eta, W0, 1, g, bt)
        assert rel(Z, Zo) < 1e-13 and rel(W, Wo) < 1e-13


# ---------------------------------------------------------------------------
# P-3: agreement with page 1's own parametrisation. Section 2 prints the online
# update W_t = W_{t-1} - eta (W_{t-1} k_t - v_t) k_t^T for f(k;W) = W k and the
# loss (1/2)||W k - v||^2; section 3 evaluates z_t = W_t q_t. With W_page = W^T
# and eta_page = 2 eta this is the oracle's row-vector, no-1/2 form.
# ---------------------------------------------------------------------------
def test_online_matches_page_update_rule(oracle_mod):
    rng = np.random.default_rng(3)
    N, d = 19, 6
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d)) / np.sqrt(d)
    v = rng.standard_normal((N, d))
    eta = rng.uniform(0.01, 0.2, N)
    W0 = rng.standard_normal((d, d)) / np.sqrt(d)
    # page form, column vectors
    Wp = W0.T.copy()
    zs = []
    for t in range(N):
        kt, vt, qt = k[t][:, None], v[t][:, None], q[t][:, None]
        Wp = Wp - (2 * eta[t]) * (Wp @ kt - vt) @ kt.T
        zs.append((Wp @ qt)[:, 0])
    Zpage = np.array(zs)
    Z, W = oracle_mod.linear(oracle_mod.ONLINE, 0, q[None, None], k[None, None], v[None, None],
                             eta[None, None], W0[None, None], 1)
    assert rel(Z[0, 0], Zpage) < 1e-13
    assert rel(W[0, 0], Wp.T) < 1e-13


# ---------------------------------------------------------------------------
# P-4: eta = 0 leaves the state untouched, so Z = f(Q; W0). f is evaluated here
# with library routines (matmul, torch layer_norm, torch's exact-erf gelu).
# ---------------------------------------------------------------------------
def _torch_f_linear(kind, Q, W0, g, bt, eps):
    Qt, Wt = torch.from_numpy(Q), torch.from_numpy(W0)
    h = Qt @ Wt
    if kind == 0:
        return h.numpy()
    H, d = g.shape
    out = torch.empty_like(h)
    for hh in range(H):
        out[:, hh] = Qt[:, hh] + torch.nn.functional.layer_norm(
            h[:, hh], (d,), torch.from_numpy(g[hh]), torch.from_numpy(bt[hh]), eps)
    return out.numpy()


@pytest.mark.parametrize("kind", [0, 1])
def test_eta_zero_linear(oracle_mod, kind):
    rng = np.random.default_rng(21)
    Q, K, V, _, W0, g, bt = rand_problem(rng, 2, 3, 21, 8)
    for mode in (0, 1, 2):
        Z, W = oracle_mod.linear(mode, kind, Q, K, V, 0.0, W0, 4, g, bt, 1e-5)
        assert np.array_equal(W, W0)
        assert rel(Z, _torch_f_linear(kind, Q, W0, g, bt, 1e-5)) < 1e-13


def test_eta_zero_mlp(oracle_mod):
    rng = np.random.default_rng(22)
    Q, K, V, _, W1, W2, g, bt = rand_problem(rng, 1, 2, 13, 4, hid=16)
    Z, W1e, W2e = oracle_mod.mlp(oracle_mod.DUAL, Q, K, V, 0.0, W1, W2, 4, g, bt, 1e-5)
    assert np.array_equal(W1e, W1) and np.array_equal(W2e, W2)
    Qt = torch.from_numpy(Q)
    a = Qt @ torch.from_numpy(W1)
    hcur = torch.nn.functional.gelu(a) @ torch.from_numpy(W2)
    ref = torch.empty_like(hcur)
    for hh in range(2):
        ref[:, hh] = Qt[:, hh] + torch.nn.functional.layer_norm(
            hcur[:, hh], (4,), torch.from_numpy(g[hh]), torch.from_numpy(bt[hh]), 1e-5)
    assert rel(Z, ref.numpy()) < 1e-13


# ---------------------------------------------------------------------------
# P-5: plain TTT-Linear from W0 = 0 in one mini-batch is unnormalised causal
# linear attention (page 1, section 4: the in-batch matrices "mirror causal
# attention"): Z = 2 tril(Q K^T) diag(eta) V and W_end = 2 K^T diag(eta) V.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,b", [(16, 16), (11, 16), (1, 1)])
def test_zero_state_single_batch_is_causal_linear_attention(oracle_mod, N, b):
    rng = np.random.default_rng(N)
    d = 8
    Q = rng.standard_normal((N, d))
    K = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    eta = rng.uniform(0.1, 0.3, N)
    A = np.tril(Q @ K.T) * eta[None, :]
    Zref = 2 * A @ V
    Wref = 2 * (K * eta[:, None]).T @ V
    for mode in (oracle_mod.MINIBATCH, oracle_mod.DUAL):
        Z, W = oracle_mod.linear(mode, 0, Q[None, None], K[None, None], V[None, None],
                                 eta[None, None], np.zeros((1, 1, d, d)), b)
        assert rel(Z[0, 0], Zref) < 1e-13
        assert rel(W[0, 0], Wref) < 1e-13


# ---------------------------------------------------------------------------
# P-6: analytic gradients against autograd-free central finite differences of
# the per-token loss (page 1, section 2 gives the closed-form gradient of the
# plain model; LN and GELU backward are checked by brute force).
# ---------------------------------------------------------------------------
def _fd(fun, X, h=1e-6):
    G = np.zeros_like(X)
    it = np.nditer(X, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        Xp, Xm = X.copy(), X.copy()
        Xp[i] += h
        Xm[i] -= h
        G[i] = (fun(Xp) - fun(Xm)) / (2 * h)
    return G


@pytest.mark.parametrize("kind", [0, 1])
def test_linear_grad_finite_differences(oracle_mod, kind):
    rng = np.random.default_rng(31 + kind)
    d = 4
    W = rng.standard_normal((d, d))
    k, v = rng.standard_normal(d), rng.standard_normal(d)
    g, bt = 1 + 0.3 * rng.standard_normal(d), 0.3 * rng.standard_normal(d)
    an = oracle_mod.linear_grad(kind, W, k, v, g, bt, 1e-5)
    fd = _fd(lambda X: oracle_mod.linear_loss(kind, X, k, v, g, bt, 1e-5), W)
    assert rel(an, fd) < 1e-6
    if kind == 0:  # closed form of page 1 section 2 (transposed, no 1/2): 2 k^T (k W - v)
        assert rel(an, 2 * np.outer(k, k @ W - v)) < 1e-14


def test_mlp_grad_finite_differences(oracle_mod):
    rng = np.random.default_rng(41)
    d, hid = 4, 16
    W1 = rng.standard_normal((d, hid)) / 2
    W2 = rng.standard_normal((hid, d)) / 4
    k, v = rng.standard_normal(d), rng.standard_normal(d)
    g, bt = 1 + 0.3 * rng.standard_normal(d), 0.3 * rng.standard_normal(d)
    a1, a2 = oracle_mod.mlp_grad(W1, W2, k, v, g, bt, 1e-5)
    f1 = _fd(lambda X: oracle_mod.mlp_loss(X, W2, k, v, g, bt, 1e-5), W1)
    f2 = _fd(lambda X: oracle_mod.mlp_loss(W1, X, k, v, g, bt, 1e-5), W2)
    assert rel(a1, f1) < 1e-6
    assert rel(a2, f2) < 1e-6


def test_mlp_grad_matches_torch_autograd(oracle_mod):
    """Second, independent check of the MLP backward: torch autograd in fp64."""
    rng = np.random.default_rng(42)
    d, hid = 8, 32
    W1 = torch.tensor(rng.standard_normal((d, hid)) / 3, requires_grad=True)
    W2 = torch.tensor(rng.standard_normal((hid, d)) / 6, requires_grad=True)
    k, v = torch.tensor(rng.standard_normal(d)), torch.tensor(rng.standard_normal(d))
    g, bt = torch.tensor(1 + 0.3 * rng.standard_normal(d)), torch.tensor(0.3 * rng.standard_normal(d))
    f = k + torch.nn.functional.layer_norm(torch.nn.functional.gelu(k @ W1) @ W2, (d,), g, bt, 1e-6)
    ((f - v) ** 2).sum().backward()
    a1, a2 = oracle_mod.mlp_grad(W1.detach().numpy(), W2.detach().numpy(), k.numpy(), v.numpy(),
                                 g.numpy(), bt.numpy(), 1e-6)
    assert rel(a1, W1.grad.numpy()) < 1e-12
    assert rel(a2, W2.grad.numpy()) < 1e-12


def test_gelu_closed_forms(oracle_mod):
    import math
    for a in (-3.0, -1.0, -0.25, 0.0, 0.5, 2.0, 4.0):
        assert oracle_mod.gelu(a) - oracle_mod.gelu(-a) == pytest.approx(a, abs=1e-15)
        ref = 0.5 * a * math.erfc(-a / math.sqrt(2.0))
        assert oracle_mod.gelu(a) == pytest.approx(ref, rel=1e-14, abs=1e-300)
        h = 1e-6
        fd = (oracle_mod.gelu(a + h) - oracle_mod.gelu(a - h)) / (2 * h)
        assert oracle_mod.gelu_prime(a) == pytest.approx(fd, abs=1e-8)
    assert oracle_mod.gelu_prime(0.0) == 0.5
    t = torch.linspace(-5, 5, 101, dtype=torch.float64)
    ref = torch.nn.functional.gelu(t).numpy()
    got = np.array([oracle_mod.gelu(float(x)) for x in t])
    assert np.max(np.abs(got - ref)) < 1e-15


# ---------------------------------------------------------------------------
# P-7: the returned state continues the sequence (the state is the layer's
# whole memory, page 1 section 3: constant O(1) state).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind", [0, 1, "mlp"])
def test_state_passing(oracle_mod, kind):
    rng = np.random.default_rng(51)
    b, N1, N2 = 4, 12, 9
    if kind == "mlp":
        Q, K, V, eta, W1, W2, g, bt = rand_problem(rng, 1, 2, N1 + N2, 4, hid=16)
        Z, W1e, W2e = oracle_mod.mlp(oracle_mod.MINIBATCH, Q, K, V, eta, W1, W2, b, g, bt)
        s = slice(None, N1)
        t = slice(N1, None)
        Za, W1a, W2a = oracle_mod.mlp(oracle_mod.DUAL, Q[:, :, s], K[:, :, s], V[:, :, s],
                                      eta[:, :, s], W1, W2, b, g, bt)
        Zb, W1b, W2b = oracle_mod.mlp(oracle_mod.DUAL, Q[:, :, t], K[:, :, t], V[:, :, t],
                                      eta[:, :, t], W1a, W2a, b, g, bt)
        assert rel(np.concatenate([Za, Zb], 2), Z) < 1e-13
        assert rel(W1b, W1e) < 1e-13 and rel(W2b, W2e) < 1e-13
        return
    Q, K, V, eta, W0, g, bt = rand_problem(rng, 2, 2, N1 + N2, 8)
    Z, We = oracle_mod.linear(oracle_mod.MINIBATCH, kind, Q, K, V, eta, W0, b, g, bt)
    s, t = slice(None, N1), slice(N1, None)
    Za, Wa = oracle_mod.linear(oracle_mod.DUAL, kind, Q[:, :, s], K[:, :, s], V[:, :, s],
                               eta[:, :, s], W0, b, g, bt)
    Zb, Wb = oracle_mod.linear(oracle_mod.DUAL, kind, Q[:, :, t], K[:, :, t], V[:, :, t],
                               eta[:, :, t], Wa, b, g, bt)
    assert rel(np.concatenate([Za, Zb], 2), Z) < 1e-13
    assert rel(Wb, We) < 1e-13


# ---------------------------------------------------------------------------
# P-8: a hand-worked example (tests/golden/hand_example_linear_d1.json).
# ---------------------------------------------------------------------------
def test_hand_example(oracle_mod):
    with open(os.path.join(HERE, "golden", "hand_example_linear_d1.json")) as f:
        ex = json.load(f)
    i = ex["inputs"]
    args = [np.array(i[n], dtype=np.float64).reshape(1, 1, -1, 1) for n in ("q", "k", "v")]
    W0 = np.array([[[[i["w0"]]]]])
    for mode in (oracle_mod.MINIBATCH, oracle_mod.DUAL):
        Z, W = oracle_mod.linear(mode, 0, *args, i["eta"], W0, i["b"])
        assert np.allclose(Z.ravel(), ex["minibatch"]["z"], rtol=0, atol=1e-15)
        assert W.item() == pytest.approx(ex["minibatch"]["w_end"], abs=1e-15)
    Z, W = oracle_mod.linear(oracle_mod.ONLINE, 0, *args, i["eta"], W0, 1)
    assert np.allclose(Z.ravel(), ex["online"]["z"], rtol=0, atol=1e-15)
    assert W.item() == pytest.approx(ex["online"]["w_end"], abs=1e-15)


# ---------------------------------------------------------------------------
# P-9: LayerNorm special cases. gamma = beta = 0 makes LN(.) = 0, so f(x) = x,
# every gradient vanishes, Z = Q and the state is unchanged. With gamma = 1,
# beta = 0 every row of Z - Q has mean 0 and variance var/(var + eps) < 1.
# ---------------------------------------------------------------------------
def test_ln_zero_affine_is_identity(oracle_mod):
    rng = np.random.default_rng(61)
    Q, K, V, eta, W0, g, bt = rand_problem(rng, 2, 2, 18, 8)
    z = np.zeros_like(g)
    Z, W = oracle_mod.linear(oracle_mod.DUAL, 1, Q, K, V, eta, W0, 4, z, z)
    assert np.array_equal(Z, Q) and np.array_equal(W, W0)
    Q, K, V, eta, W1, W2, g, bt = rand_problem(rng, 1, 2, 9, 4, hid=16)
    z = np.zeros_like(g)
    Z, W1e, W2e = oracle_mod.mlp(oracle_mod.DUAL, Q, K, V, eta, W1, W2, 4, z, z)
    assert np.array_equal(Z, Q) and np.array_equal(W1e, W1) and np.array_equal(W2e, W2)


def test_ln_unit_affine_row_moments(oracle_mod):
    rng = np.random.default_rng(62)
    Q, K, V, eta, W0, g, bt = rand_problem(rng, 1, 2, 20, 8)
    eps = 1e-3
    Z, _ = oracle_mod.linear(oracle_mod.DUAL, 1, Q, K, V, eta, W0, 4, np.ones_like(g),
                             np.zeros_like(bt), eps)
    D = Z - Q
    assert np.max(np.abs(D.mean(-1))) < 1e-14
    var = D.var(-1)
    assert np.all(var < 1.0) and np.all(var > 0.9)


# ---------------------------------------------------------------------------
# P-10: structure of plain TTT-Linear. The map (W0, V) -> (Z, W_end) is jointly
# homogeneous of degree one, and output columns are independent (permuting the
# columns of W0 and V permutes those of Z and W_end).
# ---------------------------------------------------------------------------
def test_plain_homogeneity_and_column_permutation(oracle_mod):
    rng = np.random.default_rng(71)
    Q, K, V, eta, W0, g, bt = rand_problem(rng, 1, 2, 21, 8)
    Z, W = oracle_mod.linear(oracle_mod.DUAL, 0, Q, K, V, eta, W0, 4)
    Z2, W2 = oracle_mod.linear(oracle_mod.DUAL, 0, Q, K, 2.5 * V, eta, 2.5 * W0, 4)
    assert rel(Z2, 2.5 * Z) < 1e-14 and rel(W2, 2.5 * W) < 1e-14
    p = rng.permutation(8)
    Zp, Wp = oracle_mod.linear(oracle_mod.DUAL, 0, Q, K, V[..., p], eta, W0[..., p], 4)
    assert rel(Zp, Z[..., p]) < 1e-14 and rel(Wp, W[..., p]) < 1e-14


# ---------------------------------------------------------------------------
# P-11: (sequence, head) units are independent.
# ---------------------------------------------------------------------------
def test_units_independent(oracle_mod):
    rng = np.random.default_rng(81)
    Q, K, V, eta, W0, g, bt = rand_problem(rng, 3, 2, 10, 4)
    Z, W = oracle_mod.linear(oracle_mod.DUAL, 1, Q, K, V, eta, W0, 3, g, bt)
    pb = [2, 0, 1]
    Zp, Wp = oracle_mod.linear(oracle_mod.DUAL, 1, Q[pb], K[pb], V[pb], eta[pb], W0[pb], 3, g, bt)
    assert rel(Zp, Z[pb]) < 1e-15 and rel(Wp, W[pb]) < 1e-15


# ---------------------------------------------------------------------------
# P-B: block-causal large chunks (page "Test-Time Training Done Right",
# abstract): one step per chunk with gradients at the chunk's starting weights
# (the same state recursion as the mini-batch form) and one set of weights for
# every output of the chunk, the weights before or after the chunk's step.
# ---------------------------------------------------------------------------
BLOCK_SHAPES = [(1, 2, 12, 4, 4), (2, 1, 11, 8, 3), (1, 1, 16, 8, 16), (1, 2, 9, 4, 1)]


@pytest.mark.parametrize("B,H,N,d,b", BLOCK_SHAPES)
@pytest.mark.parametrize("kind", [0, 1])
def test_block_state_equals_minibatch_state(oracle_mod, B, H, N, d, b, kind):
    """Both block modes step the state exactly as the mini-batch form does."""
    rng = np.random.default_rng(500 + N + b + kind)
    Q, K, V, eta, W0, g, bt = rand_problem(rng, B, H, N, d)
    _, Wm = oracle_mod.linear(oracle_mod.MINIBATCH, kind, Q, K, V, eta, W0, b, g, bt, 1e-6)
    for mode in (oracle_mod.BLOCK_BEFORE, oracle_mod.BLOCK_AFTER):
        _, Wb = oracle_mod.linear(mode, kind, Q, K, V, eta, W0, b, g, bt, 1e-6)
        assert rel(Wb, Wm) < 1e-12


@pytest.mark.parametrize("kind", [0, 1])
def test_block_after_b1_is_online(oracle_mod, kind):
    """With one token per chunk, outputs after the step are online GD's outputs
    (page 1, sections 2 and 3: z_t uses the weights updated with token t)."""
    rng = np.random.default_rng(41 + kind)
    Q, K, V, eta, W0, g, bt = rand_problem(rng, 1, 2, 13, 8)
    Zo, Wo = oracle_mod.linear(oracle_mod.ONLINE, kind, Q, K, V, eta, W0, 1, g, bt, 1e-6)
    Za, Wa = oracle_mod.linear(oracle_mod.BLOCK_AFTER, kind, Q, K, V, eta, W0, 1, g, bt, 1e-6)
    assert rel(Za, Zo) < 1e-12 and rel(Wa, Wo) < 1e-12


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("mode_name", ["BLOCK_BEFORE", "BLOCK_AFTER"])
def test_block_outputs_from_prefix_states(oracle_mod, kind, mode_name):
    """Chunk c's outputs are f(Q_c; W) with W the state after chunks 0..c-1
    (before) or 0..c (after): the state of a prefix run of the mini-batch form,
    evaluated through eta = 0 (which leaves W untouched and gives f(Q; W))."""
    rng = np.random.default_rng(77 + kind)
    B, H, N, d, b = 1, 2, 14, 8, 4
    Q, K, V, eta, W0, g, bt = rand_problem(rng, B, H, N, d)
    mode = getattr(oracle_mod, mode_name)
    Zb, _ = oracle_mod.linear(mode, kind, Q, K, V, eta, W0, b, g, bt, 1e-6)
    for c0 in range(0, N, b):
        c1 = min(c0 + b, N)
        upto = c0 if mode_name == "BLOCK_BEFORE" else c1
        if upto > 0:
            _, Wp = oracle_mod.linear(oracle_mod.MINIBATCH, kind, Q[:, :, :upto], K[:, :, :upto],
                                      V[:, :, :upto], eta[:, :, :upto], W0, b, g, bt, 1e-6)
        else:
            Wp = W0
        zero = np.zeros((B, H, c1 - c0))
        Zf, _ = oracle_mod.linear(oracle_mod.MINIBATCH, kind, Q[:, :, c0:c1], K[:, :, c0:c1],
                                  V[:, :, c0:c1], zero, Wp, b, g, bt, 1e-6)
        assert rel(Zb[:, :, c0:c1], Zf) < 1e-12


@pytest.mark.parametrize("kind", [0, 1])
def test_block_after_last_token_matches_dual(oracle_mod, kind):
    """The last token of a full chunk sees every token of its chunk under the
    causal mask, so the dual form's output there equals the after-step output."""
    rng = np.random.default_rng(90 + kind)
    Q, K, V, eta, W0, g, bt = rand_problem(rng, 2, 1, 15, 8)
    b = 5
    Zd, _ = oracle_mod.linear(oracle_mod.DUAL, kind, Q, K, V, eta, W0, b, g, bt, 1e-6)
    Za, _ = oracle_mod.linear(oracle_mod.BLOCK_AFTER, kind, Q, K, V, eta, W0, b, g, bt, 1e-6)
    last = [c0 + b - 1 for c0 in range(0, 15, b)]
    assert rel(Za[:, :, last], Zd[:, :, last]) < 1e-12
    # and not elsewhere (the mask matters inside the chunk)
    assert rel(Za[:, :, 0], Zd[:, :, 0]) > 1e-6


def test_block_single_chunk_closed_forms(oracle_mod):
    """Plain f, W0 = 0, one chunk: before -> Z = Q W0 = 0; after -> Z = Q (2 K^T D V)."""
    rng = np.random.default_rng(12)
    Q, K, V, eta, W0, g, bt = rand_problem(rng, 1, 1, 10, 6)
    W0 = np.zeros_like(W0)
    Zb, _ = oracle_mod.linear(oracle_mod.BLOCK_BEFORE, 0, Q, K, V, eta, W0, 10, g, bt, 1e-6)
    Za, Wa = oracle_mod.linear(oracle_mod.BLOCK_AFTER, 0, Q, K, V, eta, W0, 10, g, bt, 1e-6)
    q, k, v, e = Q[0, 0], K[0, 0], V[0, 0], eta[0, 0]
    Wc = 2.0 * k.T @ (e[:, None] * v)
    assert np.max(np.abs(Zb)) == 0.0
    assert rel(Wa[0, 0], Wc) < 1e-12
    assert rel(Za[0, 0], q @ Wc) < 1e-12


@pytest.mark.parametrize("kind", [0, 1])
def test_online_one_token_steps_compose(oracle_mod, kind):
    """A single-token decode step is the online rule applied once (page 1,
    section 2); N such steps, each from the previous state, are online GD over
    the N tokens."""
    rng = np.random.default_rng(300 + kind)
    Q, K, V, eta, W0, g, bt = rand_problem(rng, 2, 2, 6, 8)
    Zo, Wo = oracle_mod.linear(oracle_mod.ONLINE, kind, Q, K, V, eta, W0, 1, g, bt, 1e-6)
    W = W0
    for t in range(6):
        z, W = oracle_mod.linear(oracle_mod.ONLINE, kind, Q[:, :, t:t + 1], K[:, :, t:t + 1],
                                 V[:, :, t:t + 1], eta[:, :, t:t + 1], W, 1, g, bt, 1e-6)
        assert rel(z[:, :, 0], Zo[:, :, t]) < 1e-12
    assert rel(W, Wo) < 1e-12
