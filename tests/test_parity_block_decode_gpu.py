"""GPU parity of the block-causal large-chunk outputs and of the single-token
decode step with the fp64 oracle, through the C ABI, on identical seeded inputs.

Tolerance per output tensor (max|gpu - ref| / max|ref|): 1e-5 for fp32 token
streams, 2e-3 for bf16 token streams (fp32 accumulation).
"""
import numpy as np
import pytest

import oracle
from weights_ttt_layer_amd import workloads as wlm

from gpu_helpers import (TOL, check_all_units, gpu_decode, gpu_linear_block, oracle_linear, rel_err,
                         row_mean_ratio, say)

pytestmark = pytest.mark.gpu

MODES = {"before": oracle.BLOCK_BEFORE, "after": oracle.BLOCK_AFTER}


def lc(B, H, N, b, eta="const", eta_const=0.01, seed=5):
    wl = wlm.Workload(f"blk_{B}x{H}x{N}_b{b}_{eta}", "plain", "bf16", B, H, N, 128, b, eta, eta_const,
                      l2_rows=True)
    return wlm.generate(wl, seed)


@pytest.mark.parametrize("apply", ["before", "after"])
@pytest.mark.parametrize("B,H,N,b,eta", [
    (1, 2, 1024, 256, "const"),
    (2, 1, 768, 256, "sigmoid"),     # per-token step sizes
    (1, 1, 640, 256, "const"),       # short last chunk (128 tokens)
    (1, 2, 2048, 512, "const"),
    (1, 1, 256, 256, "const"),       # a single chunk
    (1, 1, 1152, 384, "sigmoid"),    # three blocks per chunk
    (1, 1, 2560, 1024, "sigmoid"),   # last chunk half as long
])
def test_block_shapes(apply, B, H, N, b, eta):
    inp = lc(B, H, N, b, eta)
    say(f"case {inp.wl.name} apply={apply}")
    z, w = gpu_linear_block(inp, apply)
    zr, wr = oracle_linear(inp, MODES[apply])
    ez, ew = rel_err(z, zr), rel_err(w, wr)
    say(f"  err Z {ez:.2e}  W_end {ew:.2e}  (tol 2e-03)")
    assert ez <= TOL["bf16"] and ew <= TOL["bf16"]


def test_block_before_first_chunk_is_q_w0():
    """The first chunk's outputs before any step are Q W0 (closed form)."""
    inp = lc(1, 1, 512, 256)
    z, _ = gpu_linear_block(inp, "before")
    Q, W0 = inp.f64("q")[0, 0, :256], inp.f64("w0")[0, 0]
    assert rel_err(z[0, 0, :256], Q @ W0) <= TOL["bf16"]


@pytest.mark.parametrize("apply", ["before", "after"])
def test_block_workload_all_units(apply):
    """The full large-chunk workload (B=1 H=16 N=32768 d=128 b=2048), launched
    whole; every head compared with the oracle run over the whole input."""
    inp = wlm.workload_inputs(4)
    say(f"case {inp.wl.name} block apply={apply} (full launch, every unit)")
    z, w = gpu_linear_block(inp, apply)
    zr, wr = oracle_linear(inp, MODES[apply])
    check_all_units(f"{inp.wl.name} {apply}", [("Z", z, zr), ("W_end", w, wr)], TOL["bf16"])


@pytest.mark.parametrize("apply", ["before", "after"])
@pytest.mark.parametrize("dtype,d,B,H,N,b,eta", [
    ("bf16", 64, 1, 2, 1000, 256, "sigmoid"),    # d = 64, ragged N
    ("f32", 128, 1, 1, 700, 256, "const"),       # fp32 streams
    ("f32", 64, 2, 1, 300, 100, "sigmoid"),      # b not a multiple of 16, blocks of 64 + 36
    ("bf16", 128, 1, 1, 32040, 2048, "const"),   # the benchmark's b with N not a multiple of 128
    ("bf16", 128, 1, 2, 400, 1000, "sigmoid"),   # a single, partial chunk
    ("f32", 64, 1, 1, 65, 65, "const"),          # the shortest large chunk, one token past a block
])
def test_block_generic_shapes(apply, dtype, d, B, H, N, b, eta):
    """Large-chunk shapes outside the chunk-parallel kernels run the generic
    kernel's block mode; the block-causal outputs against the oracle."""
    std = 1.0 / np.sqrt(d) if dtype == "f32" else 1.0
    wl = wlm.Workload(f"blkg_{dtype}_d{d}_{B}x{H}x{N}_b{b}_{eta}", "plain", dtype, B, H, N, d, b, eta, 0.01,
                      qkv_std=std, l2_rows=(dtype == "bf16"))
    inp = wlm.generate(wl, 17)
    say(f"case {wl.name} apply={apply}")
    z, w = gpu_linear_block(inp, apply)
    zr, wr = oracle_linear(inp, MODES[apply])
    ez, ew = rel_err(z, zr), rel_err(w, wr)
    say(f"  err Z {ez:.2e}  W_end {ew:.2e}  (tol {TOL[dtype]:.0e})")
    assert ez <= TOL[dtype] and ew <= TOL[dtype]


def dec(kind, dtype, B, H, N, eta, seed):
    wl = wlm.Workload(f"dec_{kind}_{dtype}_{B}x{H}x{N}_{eta}", kind, dtype, B, H, N, 64, 1, eta, 0.1)
    return wlm.generate(wl, seed)


@pytest.mark.parametrize("kind,dtype,eta", [
    ("plain", "f32", "const"), ("ln", "f32", "sigmoid"), ("ln", "bf16", "sigmoid"), ("plain", "bf16", "sigmoid"),
])
def test_decode_steps_match_online(kind, dtype, eta):
    """N successive decode steps equal online GD over the N tokens (b = 1)."""
    inp = dec(kind, dtype, 3, 5, 6, eta, seed=9)
    say(f"case {inp.wl.name}")
    z, w = gpu_decode(inp)
    zr, wr = oracle_linear(inp, oracle.ONLINE)
    ez, ew = rel_err(z, zr), rel_err(w, wr)
    say(f"  err Z {ez:.2e}  W {ew:.2e}  (tol {TOL[dtype]:.0e})")
    assert ez <= TOL[dtype] and ew <= TOL[dtype]


@pytest.mark.parametrize("B,H", [(1, 1), (7, 3), (2, 12)])
@pytest.mark.parametrize("kind,dtype", [("ln", "bf16"), ("plain", "f32")])
def test_decode_stream_counts(kind, dtype, B, H):
    """Stream counts from one to a few dozen (one wave each), constant eta."""
    inp = dec(kind, dtype, B, H, 4, "const", seed=40 + B * H)
    say(f"case {inp.wl.name}")
    z, w = gpu_decode(inp)
    zr, wr = oracle_linear(inp, oracle.ONLINE)
    ez, ew = rel_err(z, zr), rel_err(w, wr)
    say(f"  err Z {ez:.2e}  W {ew:.2e}  (tol {TOL[dtype]:.0e})")
    assert ez <= TOL[dtype] and ew <= TOL[dtype]


def test_decode_workload_all_streams():
    """The decode workload (B=64 H=12 d=64, LN, bf16), one step for all 768
    streams; every stream compared with the oracle."""
    idx = [w.name for w in wlm.WORKLOADS].index("decode_ln_bf16_B64H12_d64")
    inp = wlm.workload_inputs(idx)
    say(f"case {inp.wl.name} (every stream)")
    z, w = gpu_decode(inp)
    zr, wr = oracle_linear(inp, oracle.ONLINE)
    check_all_units(inp.wl.name, [("z", z, zr), ("W", w, wr)], TOL["bf16"])


@pytest.mark.parametrize("kind,dtype", [("ln", "bf16"), ("ln", "f32")])
def test_decode_large_row_mean(kind, dtype):
    """LayerNorm inputs whose row mean is 30-40 times their spread (the state
    offset by a constant): the decode step's centred variance must still match.
    (The step forms h = k W in fp32 from the state as given, so its absolute
    rounding grows with the row mean; at 1e-5 this holds up to a ratio of ~100.)"""
    inp = dec(kind, dtype, 2, 3, 5, "sigmoid", seed=23)
    inp.w0 = (inp.w0.astype(np.float64) + 6.0).astype(np.float32)
    ratio = row_mean_ratio(inp.f64("k"), inp.f64("w0"))
    say(f"case {inp.wl.name} (offset state): median |mean|/std of k W0 rows {ratio:.0f}")
    assert ratio >= 30.0
    z, w = gpu_decode(inp)
    zr, wr = oracle_linear(inp, oracle.ONLINE)
    ez, ew = rel_err(z, zr), rel_err(w, wr)
    say(f"  err Z {ez:.2e}  W {ew:.2e}  (tol {TOL[dtype]:.0e})")
    assert ez <= TOL[dtype] and ew <= TOL[dtype]


def test_decode_graph_replay_matches_eager():
    """Decode steps captured in a HIP graph (as the benchmark times them): each
    of several replays, with eager work and a synchronisation in between, leaves
    the same z and state as the same steps run eagerly (bit for bit: the same
    kernel on the same inputs)."""
    import torch
    from weights_ttt_layer_amd import linear_decode
    inp = dec("ln", "bf16", 4, 6, 3, "sigmoid", seed=21)
    say(f"case {inp.wl.name} (graph replay)")
    t = wlm.to_device(inp)
    wl = inp.wl
    steps = [(t["q"][:, :, i].contiguous(), t["k"][:, :, i].contiguous(), t["v"][:, :, i].contiguous(),
              t["eta"][:, :, i].contiguous()) for i in range(wl.N)]
    kw = dict(kind=wl.kind, eta_const=inp.eta_const, ln_gamma=t["gamma"], ln_beta=t["beta"], ln_eps=wl.ln_eps)
    reps = 3

    w_e = t["w0"].clone()
    ref = []
    for _ in range(reps):
        zs = [linear_decode(q, k, v, w_e, eta, **kw) for (q, k, v, eta) in steps]
        ref.append(([z.clone() for z in zs], w_e.clone()))
    torch.cuda.synchronize()

    w_g = t["w0"].clone()
    zg = [torch.empty_like(ref[0][0][0]) for _ in steps]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for (q, k, v, eta), z in zip(steps, zg):
            linear_decode(q, k, v, w_g, eta, z=z, stream=cap, **kw)
    torch.cuda.synchronize()
    assert torch.equal(w_g, t["w0"]), "capture must not run the steps"
    for r in range(reps):
        graph.replay()
        noise = torch.randn(1 << 16, device=w_g.device).square().sum()   # eager work between replays
        torch.cuda.synchronize()
        assert bool(torch.isfinite(noise))
        same_z = all(torch.equal(a, b) for a, b in zip(zg, ref[r][0]))
        same_w = torch.equal(w_g, ref[r][1])
        say(f"  replay {r}: z identical {same_z}, state identical {same_w}")
        assert same_z and same_w
