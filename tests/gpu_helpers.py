"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and
the fp64 oracle on the same seeded inputs, and measure the normwise error."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from weights_ttt_layer_amd import workloads as wlm

TOL = {"f32": 1e-5, "bf16": 2e-3}


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| over one output tensor."""
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got.astype(np.float64) - ref)))
    return num if den == 0.0 else num / den


def unit_errs(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """rel_err of every (sequence, head) unit of [B, H, ...] arrays: the maximum
    absolute difference over the unit's outputs divided by the unit's max |ref|."""
    B, H = ref.shape[:2]
    diff = np.abs(got.astype(np.float64) - ref).reshape(B, H, -1).max(axis=2)
    den = np.abs(ref).reshape(B, H, -1).max(axis=2)
    return np.where(den > 0, diff / np.where(den > 0, den, 1.0), diff)


def check_all_units(name: str, pairs, tol: float):
    """Assert every unit of every (label, got, ref) pair is within tol; print the
    worst unit of each."""
    worst = {}
    for label, got, ref in pairs:
        e = unit_errs(got, ref)
        bi, hi = np.unravel_index(int(np.argmax(e)), e.shape)
        worst[label] = (float(e.max()), (int(bi), int(hi)))
        say(f"  {name} {label}: all {e.size} units, worst {e.max():.2e} at unit ({bi},{hi}), "
            f"median {np.median(e):.2e} (tol {tol:.0e})")
    for label, (e, u) in worst.items():
        assert e <= tol, f"{name} {label}: unit {u} error {e:.2e} > {tol:.0e}"


def row_mean_ratio(x: np.ndarray, w: np.ndarray) -> float:
    """Median over the rows of h = x W of |mean(h)| / std(h), x [B,H,T,d] and
    W [B,H,d,e] in fp64: how far a LayerNorm input's mean sits above its spread."""
    h = np.einsum("bhtd,bhde->bhte", x, w)
    return float(np.median(np.abs(h.mean(-1)) / h.std(-1)))


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_linear(inp: wlm.Inputs, in_place: bool = False, **kw):
    import torch
    from weights_ttt_layer_amd import linear_fwd
    t = wlm.to_device(inp)
    wl = inp.wl
    w_end = t["w0"] if in_place else None
    z, w = linear_fwd(t["q"], t["k"], t["v"], t["w0"], t["eta"], b=wl.b, kind=wl.kind,
                      eta_const=inp.eta_const, ln_gamma=t["gamma"], ln_beta=t["beta"],
                      ln_eps=wl.ln_eps, w_end=w_end, **kw)
    torch.cuda.synchronize()
    return z.cpu().numpy(), w.cpu().numpy()


def gpu_mlp(inp: wlm.Inputs):
    import torch
    from weights_ttt_layer_amd import mlp_fwd
    t = wlm.to_device(inp)
    wl = inp.wl
    z, w1, w2 = mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], b=wl.b,
                        eta_const=inp.eta_const, ln_gamma=t["gamma"], ln_beta=t["beta"],
                        ln_eps=wl.ln_eps)
    torch.cuda.synchronize()
    return z.cpu().numpy(), w1.cpu().numpy(), w2.cpu().numpy()


def oracle_linear(inp: wlm.Inputs, mode=oracle.MINIBATCH):
    wl = inp.wl
    kind = oracle.LN if wl.kind == "ln" else oracle.PLAIN
    return oracle.linear(mode, kind, inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.eta_f64(),
                         inp.f64("w0"), wl.b,
                         None if inp.gamma is None else inp.f64("gamma"),
                         None if inp.beta is None else inp.f64("beta"), wl.ln_eps)


def oracle_mlp(inp: wlm.Inputs, mode=oracle.MINIBATCH):
    wl = inp.wl
    return oracle.mlp(mode, inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.eta_f64(), inp.f64("w1"),
                      inp.f64("w2"), wl.b, inp.f64("gamma"), inp.f64("beta"), wl.ln_eps)


def sample_units(wl: wlm.Workload, count: int, seed: int = 0):
    """A deterministic spread of (b, h) units: the first, the last, and random ones."""
    rng = np.random.default_rng(seed)
    units = {(0, 0), (wl.B - 1, wl.H - 1)}
    while len(units) < min(count, wl.B * wl.H):
        units.add((int(rng.integers(wl.B)), int(rng.integers(wl.H))))
    return sorted(units)


def gpu_linear_block(inp: wlm.Inputs, apply: str):
    import torch
    from weights_ttt_layer_amd import linear_fwd_block
    t = wlm.to_device(inp)
    wl = inp.wl
    z, w = linear_fwd_block(t["q"], t["k"], t["v"], t["w0"], t["eta"], b=wl.b, apply=apply, kind=wl.kind,
                            eta_const=inp.eta_const, ln_gamma=t["gamma"], ln_beta=t["beta"], ln_eps=wl.ln_eps)
    torch.cuda.synchronize()
    return z.cpu().numpy(), w.cpu().numpy()


def gpu_decode(inp: wlm.Inputs):
    """Run the N tokens of `inp` as N successive single-token decode steps from
    W0. Returns (Z [B,H,N,d], final W)."""
    import torch
    from weights_ttt_layer_amd import linear_decode
    t = wlm.to_device(inp)
    wl = inp.wl
    w = t["w0"].clone()
    zs = []
    for i in range(wl.N):
        eta = None if t["eta"] is None else t["eta"][:, :, i].contiguous()
        z = linear_decode(t["q"][:, :, i].contiguous(), t["k"][:, :, i].contiguous(),
                          t["v"][:, :, i].contiguous(), w, eta, kind=wl.kind, eta_const=inp.eta_const,
                          ln_gamma=t["gamma"], ln_beta=t["beta"], ln_eps=wl.ln_eps)
        zs.append(z)
    torch.cuda.synchronize()
    return torch.stack(zs, 2).cpu().numpy(), w.cpu().numpy()
