"""GPU parity of the large-chunk TTT-Linear path (plain f, d = 128, b >= 256)
with the fp64 oracle, through the C ABI, on identical seeded inputs.

Tolerance per output tensor (max|gpu - ref| / max|ref|): 2e-3 (bf16 token
streams with fp32 accumulation).
"""
import numpy as np
import pytest

from weights_ttt_layer_amd import workloads as wlm

from gpu_helpers import TOL, check_all_units, gpu_linear, oracle_linear, rel_err, say

pytestmark = pytest.mark.gpu


def lc(B, H, N, b, eta="const", eta_const=0.01, seed=5):
    wl = wlm.Workload(f"lc_{B}x{H}x{N}_b{b}_{eta}", "plain", "bf16", B, H, N, 128, b, eta, eta_const,
                      l2_rows=True)
    return wlm.generate(wl, seed)


def check(inp):
    z, w = gpu_linear(inp)
    zr, wr = oracle_linear(inp)
    ez, ew = rel_err(z, zr), rel_err(w, wr)
    say(f"  {inp.wl.name}: err Z {ez:.2e}  W_end {ew:.2e}  (tol 2e-03)")
    assert ez <= TOL["bf16"] and ew <= TOL["bf16"]


@pytest.mark.parametrize("B,H,N,b,eta", [
    (1, 2, 1024, 256, "const"),      # 4 chunks of 8 query blocks... of 2 blocks each
    (2, 1, 768, 256, "sigmoid"),     # per-token step sizes
    (1, 1, 640, 256, "const"),       # short last chunk (128 tokens)
    (1, 2, 2048, 512, "const"),      # 4 blocks per chunk
    (1, 1, 256, 256, "const"),       # a single chunk
    (1, 1, 1152, 384, "sigmoid"),    # b a multiple of 128 but not of 256: three blocks per chunk
    (1, 1, 2560, 1024, "sigmoid"),   # b = 1024, last chunk half as long
    (1, 1, 4096, 2048, "const"),     # the benchmark chunk size, every output compared
])
def test_large_chunk_shapes(B, H, N, b, eta):
    inp = lc(B, H, N, b, eta)
    say(f"case {inp.wl.name}")
    check(inp)


def test_large_chunk_single_chunk_is_causal_linear_attention():
    """W0 = 0, one chunk: Z = 2 tril(Q K^T) diag(eta) V exactly (unnormalised
    causal linear attention), W_end = 2 K^T diag(eta) V; checked through the
    oracle of record and the closed form."""
    inp = lc(1, 1, 512, 512, "const", 0.02)
    inp.w0 = np.zeros_like(inp.w0)
    z, w = gpu_linear(inp)
    Q, K, V = (inp.f64(n)[0, 0] for n in ("q", "k", "v"))
    eta = float(np.float32(0.02))
    zc = 2 * eta * np.tril(Q @ K.T) @ V
    wc = 2 * eta * K.T @ V
    assert rel_err(z[0, 0], zc) <= TOL["bf16"]
    assert rel_err(w[0, 0], wc) <= TOL["bf16"]


def test_large_chunk_workload_all_units():
    """The full large-chunk workload (B=1 H=16 N=32768 d=128 b=2048, eta = 0.01),
    launched whole (the 16-step scan of every head on its XCD-mapped grid); every
    head compared with the oracle run over the whole input."""
    inp = wlm.workload_inputs(4)
    say(f"case {inp.wl.name} (full launch, every unit)")
    z, w = gpu_linear(inp)
    zr, wr = oracle_linear(inp)
    check_all_units(inp.wl.name, [("Z", z, zr), ("W_end", w, wr)], TOL["bf16"])


def test_large_chunk_state_passing():
    """run(N1 + N2) equals run(N1) then run(N2) from the returned state (N1 % b == 0)."""
    inp = lc(1, 2, 1024, 256, "const")
    z, w = gpu_linear(inp)
    N1 = 512
    a = wlm.Inputs(inp.wl.replace(N=N1), inp.q[:, :, :N1].copy(), inp.k[:, :, :N1].copy(),
                   inp.v[:, :, :N1].copy(), None, inp.eta_const, inp.w0)
    za, wa = gpu_linear(a)
    b2 = wlm.Inputs(inp.wl.replace(N=1024 - N1), inp.q[:, :, N1:].copy(), inp.k[:, :, N1:].copy(),
                    inp.v[:, :, N1:].copy(), None, inp.eta_const, wa)
    zb, wb = gpu_linear(b2)
    assert rel_err(np.concatenate([za, zb], 2), z) <= 1e-6
    assert rel_err(wb, w) <= 1e-6


def gen_case(B, H, N, d, b, dtype="bf16", eta="const", eta_const=0.01, seed=9, l2=True):
    wl = wlm.Workload(f"lcg_{dtype}_{B}x{H}x{N}_d{d}_b{b}_{eta}", "plain", dtype, B, H, N, d, b, eta, eta_const,
                      l2_rows=l2, qkv_std=1.0 if l2 or dtype == "bf16" else 0.125)
    return wlm.generate(wl, seed)


@pytest.mark.parametrize("B,H,N,d,b,dtype,eta", [
    (1, 2, 1000, 64, 256, "bf16", "const"),     # d = 64 and N not a multiple of 128 (or of b)
    (1, 1, 1000, 128, 256, "bf16", "sigmoid"),  # d = 128 with a ragged N: outside the chunk-parallel kernels
    (2, 1, 700, 64, 256, "f32", "sigmoid"),     # fp32 streams
    (1, 1, 900, 128, 384, "f32", "const"),
    (1, 2, 350, 64, 100, "bf16", "sigmoid"),    # b between the small-b limit and 256, blocks of 64 + 36
    (1, 1, 200, 128, 65, "bf16", "const"),      # one token past the small-b limit
    (1, 1, 3000, 64, 2048, "bf16", "const"),    # b = 2048 at d = 64, a short last chunk
])
def test_large_chunk_generic(B, H, N, d, b, dtype, eta):
    """Plain TTT-Linear with chunks longer than 64 tokens outside the bf16 d = 128
    chunk-parallel kernels: the generic kernel in blocks of 64 tokens (the
    chunk-start state for the gradients, a running state for the outputs)."""
    inp = gen_case(B, H, N, d, b, dtype, eta)
    say(f"case {inp.wl.name}")
    tol = TOL[dtype]
    z, w = gpu_linear(inp)
    zr, wr = oracle_linear(inp)
    ez, ew = rel_err(z, zr), rel_err(w, wr)
    say(f"  err Z {ez:.2e}  W_end {ew:.2e}  (tol {tol:.0e})")
    assert ez <= tol and ew <= tol


def test_large_chunk_generic_single_chunk_closed_form():
    """W0 = 0, one chunk of 640 tokens at d = 64: Z = 2 tril(Q K^T) diag(eta) V,
    W_end = 2 K^T diag(eta) V (unnormalised causal linear attention)."""
    inp = gen_case(1, 1, 640, 64, 640, "bf16", "const", 0.02, seed=10)
    inp.w0 = np.zeros_like(inp.w0)
    z, w = gpu_linear(inp)
    Q, K, V = (inp.f64(n)[0, 0] for n in ("q", "k", "v"))
    eta = float(np.float32(0.02))
    assert rel_err(z[0, 0], 2 * eta * np.tril(Q @ K.T) @ V) <= TOL["bf16"]
    assert rel_err(w[0, 0], 2 * eta * K.T @ V) <= TOL["bf16"]
