"""GPU parity of the small-b TTT-Linear path (plain and LayerNorm+residual) with
the fp64 oracle, through the C ABI, on identical seeded inputs.

Tolerance (per output tensor, max|gpu - ref| / max|ref|): 1e-5 for fp32 token
streams, 2e-3 for bf16 token streams with fp32 accumulation.
"""
import numpy as np
import pytest

import oracle
from weights_ttt_layer_amd import workloads as wlm

from gpu_helpers import TOL, check_all_units, gpu_linear, oracle_linear, rel_err, say

pytestmark = pytest.mark.gpu


def small(kind, dtype, B, H, N, b, eta="sigmoid", seed=7, **kw):
    wl = wlm.Workload(f"edge_{kind}_{dtype}_{B}x{H}x{N}_b{b}", kind, dtype, B, H, N, 64, b, eta,
                      0.05, qkv_std=1.0 if dtype == "bf16" else 0.125, **kw)
    return wlm.generate(wl, seed)


def check(inp, tol=None, in_place=False):
    tol = tol or TOL[inp.wl.dtype]
    z, w = gpu_linear(inp, in_place=in_place)
    zr, wr = oracle_linear(inp)
    ez, ew = rel_err(z, zr), rel_err(w, wr)
    say(f"  {inp.wl.name}: err Z {ez:.2e}  W_end {ew:.2e}  (tol {tol:.0e})")
    assert ez <= tol and ew <= tol
    return z, w


def test_workload_linear_f32_B1H1N256():
    """TTT-Linear, fp32, B=1 H=1 N=256 d=64 b=16, eta = 0.1: full comparison."""
    inp = wlm.workload_inputs(0)
    say(f"case {inp.wl.name}")
    check(inp)


CASES = [
    (kind, dtype, B, H, N, b)
    for kind in ("plain", "ln")
    for dtype in ("f32", "bf16")
    for (B, H, N, b) in [(2, 3, 37, 16), (1, 2, 5, 16), (1, 1, 100, 1), (2, 1, 64, 3),
                         (1, 1, 1, 16), (3, 2, 129, 7)]
]


@pytest.mark.parametrize("kind,dtype,B,H,N,b", CASES)
def test_edge_shapes(kind, dtype, B, H, N, b):
    """Ragged tails (N % b != 0), N < b, b = 1 (online GD), odd b, one token."""
    inp = small(kind, dtype, B, H, N, b)
    say(f"case {inp.wl.name}")
    check(inp)


@pytest.mark.parametrize("b", range(1, 17))
@pytest.mark.parametrize("kind,dtype", [("plain", "bf16"), ("ln", "bf16"), ("plain", "f32"), ("ln", "f32")])
def test_every_chunk_size(kind, dtype, b):
    """Every chunk size the small-b path takes (1 <= b <= 16), on both kernels
    (bf16 and fp32 streams): three full chunks and a ragged tail of b // 2 + 1
    tokens (a full chunk when b = 1), two units, per-token eta."""
    N = 3 * b + b // 2 + 1
    inp = small(kind, dtype, 1, 2, N, b, seed=100 + b)
    say(f"case {inp.wl.name}")
    check(inp)


@pytest.mark.parametrize("index", [1, 2])
def test_workload_ln_bf16_all_units(index):
    """Full-size LN workloads (B=8 H=12 N=2048; B=16 H=12 N=8192), launched whole
    exactly as the benchmark launches them; every output of every unit is
    compared with the oracle run over the whole input."""
    inp = wlm.workload_inputs(index)
    say(f"case {inp.wl.name} (full launch, every unit)")
    z, w = gpu_linear(inp)
    zr, wr = oracle_linear(inp)
    check_all_units(inp.wl.name, [("Z", z, zr), ("W_end", w, wr)], TOL["bf16"])


def offset_state(inp, c: float):
    """Add c to every entry of W0: each pre-activation row k W0 gains c * sum(k),
    a row mean far above the row's spread (LayerNorm's cancellation case)."""
    inp.w0 = (inp.w0.astype(np.float64) + c).astype(np.float32)
    return inp


def mean_to_spread(inp):
    """Median and 10th percentile over the first chunk's key rows of
    |mean(k W0)| / std(k W0) (the ratio the offset cases aim at)."""
    h = np.einsum("bhtd,bhde->bhte", inp.f64("k")[:, :, :inp.wl.b], inp.f64("w0"))
    r = np.abs(h.mean(-1)) / h.std(-1)
    return float(np.median(r)), float(np.percentile(r, 10))


@pytest.mark.parametrize("dtype,c", [("bf16", 6.0), ("bf16", 60.0), ("f32", 6.0), ("f32", 60.0)])
def test_ln_large_row_mean(dtype, c):
    """LayerNorm inputs whose row mean is 30-300 times their spread: the state is
    offset by a constant c, so every pre-activation row (keys and queries) gets a
    large common shift. A variance formed as E[h^2] - mu^2 would cancel
    catastrophically here; the kernels must still match the oracle."""
    inp = offset_state(small("ln", dtype, 2, 3, 90, 16, seed=31), c)
    med, p10 = mean_to_spread(inp)
    say(f"case {inp.wl.name} offset {c}: |mean|/std of k W0 rows: median {med:.0f}, 10th pct {p10:.0f}")
    assert med >= 30.0
    check(inp)


@pytest.mark.parametrize("kind,dtype", [("plain", "f32"), ("ln", "bf16")])
def test_eta_zero_gives_f_of_q(kind, dtype):
    """eta = 0 leaves the state untouched: W_end = W0 exactly, Z = f(Q; W0)."""
    inp = small(kind, dtype, 2, 2, 40, 16, eta="const")
    inp.eta_const = 0.0
    z, w = gpu_linear(inp)
    assert np.array_equal(w, inp.w0)
    zr, _ = oracle_linear(inp)
    assert rel_err(z, zr) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ln_zero_affine_gives_identity(dtype):
    """gamma = beta = 0: LN(.) = 0, so Z = Q exactly and the state is unchanged."""
    inp = small("ln", dtype, 1, 3, 50, 16)
    inp.gamma = np.zeros_like(inp.gamma)
    inp.beta = np.zeros_like(inp.beta)
    z, w = gpu_linear(inp)
    assert np.array_equal(z, inp.f64("q").astype(np.float32))
    assert np.array_equal(w, inp.w0)


@pytest.mark.parametrize("kind", ["plain", "ln"])
def test_state_passing(kind):
    """run(N1 + N2) equals run(N1) followed by run(N2) from the returned state,
    up to rounding: an uninterrupted run forms the pre-activation of the chunk
    after the split as K_c W_{c-1} - (K_c K_{c-1}^T) Gt_{c-1}, a restarted one
    as K_c W_c. Each run is within ~5e-6 of the oracle (two-term operands,
    2^-16 per entry), so the two differ by at most the sum of those errors."""
    inp = small(kind, "bf16", 2, 2, 96, 16)
    z, w = gpu_linear(inp)
    N1 = 48
    a = wlm.Inputs(inp.wl.replace(N=N1), inp.q[:, :, :N1], inp.k[:, :, :N1], inp.v[:, :, :N1],
                   inp.eta[:, :, :N1], inp.eta_const, inp.w0, None, None, inp.gamma, inp.beta)
    za, wa = gpu_linear(a)
    b2 = wlm.Inputs(inp.wl.replace(N=96 - N1), inp.q[:, :, N1:].copy(), inp.k[:, :, N1:].copy(),
                    inp.v[:, :, N1:].copy(), inp.eta[:, :, N1:].copy(), inp.eta_const, wa, None,
                    None, inp.gamma, inp.beta)
    zb, wb = gpu_linear(b2)
    assert rel_err(np.concatenate([za, zb], 2), z) <= 2e-5
    assert rel_err(wb, w) <= 2e-5


def test_in_place_state_and_determinism():
    """W_end may alias W0; two identical launches give bitwise identical outputs."""
    inp = small("ln", "bf16", 2, 3, 77, 16)
    z1, w1 = gpu_linear(inp)
    z2, w2 = gpu_linear(inp, in_place=True)
    assert np.array_equal(z1, z2) and np.array_equal(w1, w2)


def test_units_independent():
    """Permuting the batch permutes the outputs (units never interact)."""
    inp = small("ln", "bf16", 3, 2, 33, 16)
    z, w = gpu_linear(inp)
    p = [2, 0, 1]
    perm = wlm.Inputs(inp.wl, inp.q[p].copy(), inp.k[p].copy(), inp.v[p].copy(), inp.eta[p].copy(),
                      inp.eta_const, inp.w0[p].copy(), None, None, inp.gamma, inp.beta)
    zp, wp = gpu_linear(perm)
    assert np.array_equal(zp, z[p]) and np.array_equal(wp, w[p])
