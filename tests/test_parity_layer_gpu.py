"""GPU parity of the whole layer (ttt_layer_fwd: projections, key normalisation,
inner TTT-Linear, output LayerNorm + residual + W_O) with the fp64 oracle, on
identical seeded inputs (bf16 x and projection weights, fp32 state).

Tolerances (max|gpu - ref| / max|ref| per tensor):
  * Q, K, V: 1e-5 -- exact bf16 products summed in fp32, stored as two bf16
    terms (RNE rounding and the rounding of the remainder: at most 2^-18
    relative per entry).
  * Z, W_end: 2e-5 -- the inner model carries the fp32 projected streams, the
    state and the gradients as two bf16 terms (16 significant bits, at most
    2^-16 relative per operand entry), products keeping the term pairs i+j < 2.
  * y: 2e-5 -- LayerNorm(z) + q enters W_O's product as two bf16 terms, the
    same 2^-16 per entry; summed over H*d products with independent signs it
    stays near 1e-5 of max|y|.
"""
import numpy as np
import pytest

import oracle
from weights_ttt_layer_amd import workloads as wlm

from gpu_helpers import check_all_units, rel_err, say

pytestmark = pytest.mark.gpu

TOL = {"Q": 1e-5, "K": 1e-5, "V": 1e-5, "Z": 2e-5, "W_end": 2e-5, "y": 2e-5}


def oracle_layer(inp: wlm.LayerInputs, seqs=None):
    wl = inp.wl
    sl = slice(None) if seqs is None else seqs
    kind = oracle.LN if wl.kind == "ln" else oracle.PLAIN
    return oracle.layer(kind, inp.f64("x")[sl], inp.f64("wq"), inp.f64("wk"), inp.f64("wv"),
                        inp.f64("wo"), inp.f64("eta")[sl], inp.f64("w0")[sl], wl.b, wl.H,
                        inp.f64("gamma"), inp.f64("beta"), inp.f64("gamma_o"), inp.f64("beta_o"),
                        wl.ln_eps)


def gpu_layer(inp: wlm.LayerInputs, in_place=False, eta_none=False):
    import torch
    from weights_ttt_layer_amd import layer_fwd, layer_parts
    wl = inp.wl
    t = wlm.layer_to_device(inp)
    y, we, ws = layer_fwd(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], t["w0"], t["gamma_o"],
                          t["beta_o"], None if eta_none else t["eta"], H=wl.H, b=wl.b, kind=wl.kind,
                          eta_const=0.0, ln_gamma=t["gamma"], ln_beta=t["beta"], ln_eps=wl.ln_eps,
                          w_end=t["w0"] if in_place else None)
    torch.cuda.synchronize()
    parts = {k: v.cpu().numpy() for k, v in layer_parts(ws, wl.B, wl.N, wl.H, wl.d).items()}
    return y.cpu().numpy(), we.cpu().numpy(), parts


def check(inp, y, we, parts, ref, seqs=slice(None)):
    yr, wr, pr = ref
    errs = {name: rel_err(parts[name][seqs], pr[name]) for name in "QKVZ"}
    errs["W_end"] = rel_err(we[seqs], wr)
    errs["y"] = rel_err(y[seqs], yr)
    say("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL[k], k


def case(kind, B, N, D, H, b, seed=3):
    wl = wlm.LayerWorkload(f"layer_{kind}_B{B}N{N}_D{D}_H{H}_b{b}", kind, B, N, D, H, 64, b)
    return wlm.generate_layer(wl, seed)


@pytest.mark.parametrize("kind,B,N,D,H,b", [
    ("ln", 2, 200, 128, 2, 16),      # ragged token tile (200 = 128 + 72) and chunk tail (200 % 16 = 8)
    ("plain", 1, 64, 192, 3, 16),    # odd H: the last projection tile is half full; D not a multiple of 256
    ("ln", 3, 37, 64, 1, 5),         # one head, D = 64, short ragged sequences
    ("plain", 1, 300, 512, 8, 1),    # b = 1 (online steps)
    ("ln", 2, 256, 768, 12, 16),     # the model width of the named workload
    ("ln", 1, 1, 128, 2, 16),        # a single token
    ("plain", 1, 130, 1024, 16, 16), # H = 16, D = 1024
    ("ln", 1, 77, 256, 4, 3),        # b = 3, ragged tail of 2
    ("plain", 2, 90, 256, 4, 8),     # b = 8
    ("ln", 1, 140, 384, 6, 11),      # b = 11, D = 384 (six heads)
])
def test_layer_shapes(kind, B, N, D, H, b):
    inp = case(kind, B, N, D, H, b)
    say(f"case {inp.wl.name}")
    y, we, parts = gpu_layer(inp)
    check(inp, y, we, parts, oracle_layer(inp))


def test_layer_in_place_state_and_constant_eta():
    """W_end == W0 updates the state in place; eta = NULL uses eta_const (0 here:
    the state must come back unchanged and z = f(q; W0))."""
    inp = case("ln", 1, 96, 128, 2, 16, seed=4)
    y, we, parts = gpu_layer(inp, in_place=True, eta_none=True)
    ref = oracle.layer(oracle.LN, inp.f64("x"), inp.f64("wq"), inp.f64("wk"), inp.f64("wv"),
                       inp.f64("wo"), 0.0, inp.f64("w0"), 16, 2, inp.f64("gamma"), inp.f64("beta"),
                       inp.f64("gamma_o"), inp.f64("beta_o"), 1e-6)
    check(inp, y, we, parts, ref)
    assert rel_err(we, inp.w0.astype(np.float64)) <= 1e-7


def test_layer_zero_input_token():
    """A token whose x is zero has a zero key (no NaN from the normalisation)."""
    inp = case("plain", 1, 48, 128, 2, 16, seed=6)
    inp.x[0, 7, :] = 0
    y, we, parts = gpu_layer(inp)
    assert np.all(np.isfinite(y))
    assert np.all(parts["K"][0, :, 7, :] == 0)
    check(inp, y, we, parts, oracle_layer(inp))


def test_layer_named_workload_all_sequences():
    """The named workload at full size, in the launch configuration the
    benchmark times; all eight sequences checked against the oracle run over
    the whole input."""
    inp = wlm.layer_workload_inputs(0)
    say(f"case {inp.wl.name} (every sequence)")
    y, we, parts = gpu_layer(inp)
    yr, wr, pr = oracle_layer(inp)
    pairs = [(k, parts[k], pr[k]) for k in "QKVZ"] + [("W_end", we, wr)]
    for label, got, ref in pairs:
        check_all_units(inp.wl.name, [(label, got, ref)], TOL[label])
    # y is [B, N, D]: per sequence
    for s in range(inp.wl.B):
        e = rel_err(y[s], yr[s])
        say(f"  sequence {s}: y {e:.2e}")
        assert e <= TOL["y"]


def test_layer_large_row_mean():
    """Inner LayerNorm inputs whose row mean is far above their spread (W0 offset
    by a constant): the chain kernel on two-term streams must still match."""
    inp = case("ln", 1, 96, 128, 2, 16, seed=8)
    inp.w0 = (inp.w0.astype(np.float64) + 6.0).astype(np.float32)
    say(f"case {inp.wl.name} (offset state)")
    y, we, parts = gpu_layer(inp)
    check(inp, y, we, parts, oracle_layer(inp))
