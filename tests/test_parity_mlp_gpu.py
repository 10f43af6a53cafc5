"""GPU parity of the TTT-MLP path (f(x) = x + LN(GELU(x W1) W2)) with the fp64
oracle, through the C ABI, on identical seeded inputs.

Tolerance per output tensor (max|gpu - ref| / max|ref|): 1e-5 for fp32 token
streams, 2e-3 for bf16 token streams.
"""
import numpy as np
import pytest

from weights_ttt_layer_amd import workloads as wlm

from gpu_helpers import TOL, gpu_mlp, oracle_mlp, rel_err, sample_units, say

pytestmark = pytest.mark.gpu


def small(dtype, B, H, N, b, eta="sigmoid", seed=11):
    wl = wlm.Workload(f"mlp_{dtype}_{B}x{H}x{N}_b{b}", "mlp", dtype, B, H, N, 64, b, eta, 0.05,
                      qkv_std=1.0 if dtype == "bf16" else 0.125)
    return wlm.generate(wl, seed)


def check(inp):
    tol = TOL[inp.wl.dtype]
    z, w1, w2 = gpu_mlp(inp)
    zr, w1r, w2r = oracle_mlp(inp)
    errs = rel_err(z, zr), rel_err(w1, w1r), rel_err(w2, w2r)
    say(f"  {inp.wl.name}: err Z {errs[0]:.2e} W1 {errs[1]:.2e} W2 {errs[2]:.2e} (tol {tol:.0e})")
    assert max(errs) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,N,b", [(2, 2, 37, 16), (1, 1, 5, 16), (1, 2, 50, 1), (2, 1, 67, 6)])
def test_mlp_edge_shapes(dtype, B, H, N, b):
    inp = small(dtype, B, H, N, b)
    say(f"case {inp.wl.name}")
    check(inp)


@pytest.mark.parametrize("b", [2, 3, 5, 8, 11, 13, 15])
def test_mlp_chunk_sizes(b):
    """Chunk sizes between the edge cases above, bf16 streams: three full chunks
    and a ragged tail, two units."""
    inp = small("bf16", 1, 2, 3 * b + b // 2 + 1, b, seed=200 + b)
    say(f"case {inp.wl.name}")
    check(inp)


def test_mlp_workload_sampled_units():
    """Full-size TTT-MLP workload (B=4 H=12 N=4096), launched whole; a spread of
    units compared with the oracle run on those units alone."""
    inp = wlm.workload_inputs(3)
    say(f"case {inp.wl.name} (full launch, sampled units)")
    z, w1, w2 = gpu_mlp(inp)
    assert np.all(np.isfinite(z))
    for (bi, hi) in sample_units(inp.wl, 3, seed=3):
        zr, w1r, w2r = oracle_mlp(inp.unit(bi, hi))
        errs = (rel_err(z[bi, hi], zr[0, 0]), rel_err(w1[bi, hi], w1r[0, 0]),
                rel_err(w2[bi, hi], w2r[0, 0]))
        say(f"  unit ({bi},{hi}): err Z {errs[0]:.2e} W1 {errs[1]:.2e} W2 {errs[2]:.2e}")
        assert max(errs) <= TOL["bf16"]


def test_mlp_zero_affine_identity():
    """gamma = beta = 0: Z = Q exactly and both weights are unchanged."""
    inp = small("bf16", 1, 2, 40, 16)
    inp.gamma = np.zeros_like(inp.gamma)
    inp.beta = np.zeros_like(inp.beta)
    z, w1, w2 = gpu_mlp(inp)
    assert np.array_equal(z, inp.f64("q").astype(np.float32))
    assert np.array_equal(w1, inp.w1) and np.array_equal(w2, inp.w2)


def test_mlp_eta_zero():
    """eta = 0: the weights are unchanged and Z = f(Q; W1_0, W2_0)."""
    inp = small("bf16", 1, 2, 40, 16, eta="const")
    inp.eta_const = 0.0
    z, w1, w2 = gpu_mlp(inp)
    assert np.array_equal(w1, inp.w1) and np.array_equal(w2, inp.w2)
    zr, _, _ = oracle_mlp(inp)
    assert rel_err(z, zr) <= TOL["bf16"]
