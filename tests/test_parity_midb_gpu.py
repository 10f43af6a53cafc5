"""GPU parity of the small-b TTT-Linear path beyond the two specialised kernels:
chunks of 17..64 tokens at head dimension 64, and head dimension 128 with
chunks of 1..64 tokens (the generic kernel), plain and LayerNorm+residual, fp32
and bf16 token streams, against the fp64 oracle through the C ABI.

Tolerance per output tensor (max|gpu - ref| / max|ref|): 1e-5 for fp32 token
streams, 2e-3 for bf16 token streams (fp32 accumulation).
"""
import numpy as np
import pytest

from weights_ttt_layer_amd import workloads as wlm

from gpu_helpers import TOL, gpu_linear, oracle_linear, rel_err, row_mean_ratio, say

pytestmark = pytest.mark.gpu


def case(kind, dtype, B, H, N, d, b, eta="sigmoid", seed=7):
    wl = wlm.Workload(f"midb_{kind}_{dtype}_{B}x{H}x{N}_d{d}_b{b}", kind, dtype, B, H, N, d, b, eta, 0.05,
                      qkv_std=1.0 if dtype == "bf16" else 0.125)
    return wlm.generate(wl, seed)


def check(inp, in_place=False):
    tol = TOL[inp.wl.dtype]
    z, w = gpu_linear(inp, in_place=in_place)
    zr, wr = oracle_linear(inp)
    ez, ew = rel_err(z, zr), rel_err(w, wr)
    say(f"  {inp.wl.name}: err Z {ez:.2e}  W_end {ew:.2e}  (tol {tol:.0e})")
    assert ez <= tol and ew <= tol
    return z, w


@pytest.mark.parametrize("b", [17, 24, 32, 40, 48, 64])
@pytest.mark.parametrize("kind,dtype", [("plain", "bf16"), ("ln", "bf16"), ("plain", "f32"), ("ln", "f32")])
def test_d64_chunks_17_to_64(kind, dtype, b):
    """Head dim 64, chunks of 17..64 tokens: three full chunks and a ragged tail
    of b // 2 + 1 tokens, two units, per-token eta."""
    inp = case(kind, dtype, 1, 2, 3 * b + b // 2 + 1, 64, b, seed=500 + b)
    say(f"case {inp.wl.name}")
    check(inp)


@pytest.mark.parametrize("b", [1, 5, 16, 20, 33, 64])
@pytest.mark.parametrize("kind,dtype", [("plain", "bf16"), ("ln", "bf16"), ("plain", "f32"), ("ln", "f32")])
def test_d128_chunks(kind, dtype, b):
    """Head dim 128, chunks of 1..64 tokens: full chunks and a ragged tail, two units."""
    N = 3 * b + b // 2 + 1 if b > 1 else 40
    inp = case(kind, dtype, 1, 2, N, 128, b, seed=600 + b)
    say(f"case {inp.wl.name}")
    check(inp)


@pytest.mark.parametrize("kind,dtype,B,H,N,d,b", [
    ("ln", "bf16", 2, 3, 30, 64, 64),     # one short chunk (N < b)
    ("plain", "f32", 1, 1, 1, 128, 64),   # a single token
    ("ln", "f32", 3, 1, 129, 128, 32),    # one-token tail
    ("plain", "bf16", 2, 2, 200, 128, 48),
    ("ln", "bf16", 1, 4, 256, 128, 16),   # the b = 16 shape at d = 128
])
def test_edge_shapes(kind, dtype, B, H, N, d, b):
    inp = case(kind, dtype, B, H, N, d, b, seed=11)
    say(f"case {inp.wl.name}")
    check(inp)


@pytest.mark.parametrize("d,b", [(64, 32), (128, 64)])
def test_in_place_and_eta_zero(d, b):
    """W_end may alias W0; eta = 0 leaves the state bit for bit and gives f(Q; W0)."""
    inp = case("ln", "bf16", 2, 2, 100, d, b, seed=13)
    z1, w1 = check(inp)
    z2, w2 = gpu_linear(inp, in_place=True)
    assert np.array_equal(z1, z2) and np.array_equal(w1, w2)
    inp0 = case("ln", "bf16", 2, 2, 100, d, b, eta="const", seed=13)
    inp0.eta_const = 0.0
    z, w = gpu_linear(inp0)
    assert np.array_equal(w, inp0.w0)
    zr, _ = oracle_linear(inp0)
    assert rel_err(z, zr) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ln_large_row_mean_d128(dtype):
    """LayerNorm inputs whose row mean is far above their spread at d = 128, b = 64
    (the state offset by a constant)."""
    inp = case("ln", dtype, 1, 2, 150, 128, 64, seed=17)
    c = 6.0 if dtype == "bf16" else 60.0
    inp.w0 = (inp.w0.astype(np.float64) + c).astype(np.float32)
    ratio = row_mean_ratio(inp.f64("k")[:, :, :64], inp.f64("w0"))
    say(f"case {inp.wl.name} offset {c}: median |mean|/std of k W0 rows {ratio:.0f}")
    assert ratio >= 30.0
    check(inp)


def test_state_passing_d128():
    """run(N1 + N2) equals run(N1) then run(N2) from the returned state (N1 % b == 0)."""
    inp = case("ln", "bf16", 1, 2, 192, 128, 32, seed=19)
    z, w = gpu_linear(inp)
    N1 = 96
    a = wlm.Inputs(inp.wl.replace(N=N1), inp.q[:, :, :N1], inp.k[:, :, :N1], inp.v[:, :, :N1],
                   inp.eta[:, :, :N1], inp.eta_const, inp.w0, None, None, inp.gamma, inp.beta)
    za, wa = gpu_linear(a)
    b2 = wlm.Inputs(inp.wl.replace(N=192 - N1), inp.q[:, :, N1:].copy(), inp.k[:, :, N1:].copy(),
                    inp.v[:, :, N1:].copy(), inp.eta[:, :, N1:].copy(), inp.eta_const, wa, None, None,
                    inp.gamma, inp.beta)
    zb, wb = gpu_linear(b2)
    assert rel_err(np.concatenate([za, zb], 2), z) <= 2e-5
    assert rel_err(wb, w) <= 2e-5
