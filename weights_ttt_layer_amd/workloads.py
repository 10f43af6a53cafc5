"""Seeded synthetic inputs for the TTT-layer forward pass.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the layer's arithmetic, so both the HIP path and the fp64 oracle
may consume what it produces.

Recipe (the same for every workload):
  * numpy ``Generator(PCG64(seed))``; the named workloads use
    ``seed = 20261203 + index``.
  * Draw order: Q, K, V, then W0 (or W1, W2), then u (per-token step sizes),
    then gamma, beta. Every draw is fp64, scaled, then rounded to fp32
    (round-to-nearest-even), then to bf16 (round-to-nearest-even) when the
    token streams are bf16. Both sides consume the rounded values.
  * ``N(0, 1/n)`` means variance 1/n; ``N(0, 0.02)`` for gamma/beta means
    standard deviation 0.02.
  * Per-token step size: eta_t = sigmoid(u_t) / d with u_t ~ N(0,1), one
    independent draw per (batch, head, token), stored fp32 [B,H,N].
  * The large-chunk workload L2-normalises every Q/K/V row in fp64 before
    rounding.

Whole-layer workloads (``LAYER_WORKLOADS``, seed ``20261303 + index``) draw, in
this order: x ~ N(0,1) [B,N,D]; W_Q, W_K, W_V ~ N(0, 1/D) [H*d, D];
W_O ~ N(0, 1/(H*d)) [D, H*d] (all rounded to bf16); W0 ~ N(0, 1/d) fp32;
u ~ N(0,1) [B,H,N] with eta = sigmoid(u) / d; then for the LN inner model its
gamma, beta; then the output LayerNorm's gamma_o, beta_o (same laws as gamma,
beta).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED_BASE = 20261203


# --------------------------------------------------------------------------
# dtype helpers
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of a stored array (fp32 values or bf16 bit patterns)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# workload description
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "plain" | "ln" | "mlp"
    dtype: str           # storage dtype of Q/K/V: "f32" | "bf16"
    B: int
    H: int
    N: int
    d: int
    b: int
    eta: str             # "const" | "sigmoid"
    eta_const: float = 0.0
    qkv_std: float = 1.0          # std of Q/K/V entries before rounding
    l2_rows: bool = False         # L2-normalise Q/K/V rows
    hidden_mult: int = 4          # MLP hidden width = hidden_mult * d
    ln_eps: float = 1e-6
    description: str = ""

    @property
    def hidden(self) -> int:
        return self.hidden_mult * self.d

    @property
    def units(self) -> int:
        return self.B * self.H

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The named workloads. Index i uses seed SEED_BASE + i. The first five are the
# forward-pass workloads; the last is the single-token decode step.
WORKLOADS = [
    Workload("linear_f32_B1H1N256_d64_b16", "plain", "f32", 1, 1, 256, 64, 16, "const", 0.1,
             qkv_std=1.0 / 8.0,
             description="TTT-Linear f(x)=xW, fp32, B=1 H=1 N=256 d=64 b=16, eta=0.1"),
    Workload("linear_ln_bf16_B8H12N2048_d64_b16", "ln", "bf16", 8, 12, 2048, 64, 16, "sigmoid",
             description="TTT-Linear f(x)=x+LN(xW), bf16 Q/K/V, B=8 H=12 N=2048 d=64 b=16, "
                         "per-token eta"),
    Workload("linear_ln_bf16_B16H12N8192_d64_b16", "ln", "bf16", 16, 12, 8192, 64, 16, "sigmoid",
             description="long-context TTT-Linear+LN, bf16, B=16 H=12 N=8192 d=64 b=16"),
    Workload("mlp_bf16_B4H12N4096_d64_b16", "mlp", "bf16", 4, 12, 4096, 64, 16, "sigmoid",
             description="TTT-MLP f(x)=x+LN(GELU(xW1)W2), W1 d x 4d, W2 4d x d, bf16, "
                         "B=4 H=12 N=4096 d=64 b=16"),
    Workload("linear_bf16_B1H16N32768_d128_b2048", "plain", "bf16", 1, 16, 32768, 128, 2048,
             "const", 0.01, l2_rows=True,
             description="large-chunk TTT-Linear, bf16 L2-normalised rows, B=1 H=16 N=32768 "
                         "d=128 b=2048, eta=0.01"),
    Workload("decode_ln_bf16_B64H12_d64", "ln", "bf16", 64, 12, 1, 64, 1, "sigmoid",
             description="single-token decode step of TTT-Linear+LN for B*H = 768 streams, bf16 "
                         "q/k/v, d=64, per-token eta (inputs drawn as the B=8 H=12 workload's)"),
]

BY_NAME = {w.name: w for w in WORKLOADS}


@dataclass
class Inputs:
    """Rounded inputs. q/k/v hold fp32 values (dtype f32) or bf16 bit patterns (uint16)."""
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    eta: Optional[np.ndarray]            # fp32 [B,H,N] or None (then eta_const)
    eta_const: float
    w0: Optional[np.ndarray] = None      # fp32 [B,H,d,d]
    w1: Optional[np.ndarray] = None      # fp32 [B,H,d,hid]
    w2: Optional[np.ndarray] = None      # fp32 [B,H,hid,d]
    gamma: Optional[np.ndarray] = None   # fp32 [H,d]
    beta: Optional[np.ndarray] = None    # fp32 [H,d]
    extra: dict = field(default_factory=dict)

    # exact fp64 views for the oracle
    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if name in ("q", "k", "v"):
            return storage_to_f64(a, self.wl.dtype)
        return np.asarray(a, dtype=np.float64)

    def eta_f64(self) -> np.ndarray:
        if self.eta is None:
            wl = self.wl
            return np.full((wl.B, wl.H, wl.N), np.float64(np.float32(self.eta_const)))
        return self.eta.astype(np.float64)

    def unit(self, bi: int, hi: int) -> "Inputs":
        """The inputs of one (sequence, head) unit as a B=1, H=1 problem."""
        sl = (slice(bi, bi + 1), slice(hi, hi + 1))
        sub = Inputs(
            self.wl.replace(B=1, H=1),
            self.q[sl], self.k[sl], self.v[sl],
            None if self.eta is None else self.eta[sl],
            self.eta_const,
            None if self.w0 is None else self.w0[sl],
            None if self.w1 is None else self.w1[sl],
            None if self.w2 is None else self.w2[sl],
            None if self.gamma is None else self.gamma[hi:hi + 1],
            None if self.beta is None else self.beta[hi:hi + 1],
        )
        return sub


def _round_store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    return x32


def generate(wl: Workload, seed: int) -> Inputs:
    """Draw the inputs of ``wl`` from ``PCG64(seed)`` in the documented order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    shape = (B, H, N, d)
    streams = []
    for _ in range(3):
        x = rng.standard_normal(shape) * wl.qkv_std
        if wl.l2_rows:
            nrm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
            x = x / np.where(nrm > 0, nrm, 1.0)
        streams.append(_round_store(x, wl.dtype))
    q, k, v = streams
    w0 = w1 = w2 = None
    if wl.kind == "mlp":
        hid = wl.hidden
        w1 = (rng.standard_normal((B, H, d, hid)) / np.sqrt(d)).astype(np.float32)
        w2 = (rng.standard_normal((B, H, hid, d)) / np.sqrt(hid)).astype(np.float32)
    else:
        w0 = (rng.standard_normal((B, H, d, d)) / np.sqrt(d)).astype(np.float32)
    eta = None
    if wl.eta == "sigmoid":
        u = rng.standard_normal((B, H, N))
        eta = (1.0 / (1.0 + np.exp(-u)) / d).astype(np.float32)
    gamma = beta = None
    if wl.kind in ("ln", "mlp"):
        gamma = (1.0 + 0.02 * rng.standard_normal((H, d))).astype(np.float32)
        beta = (0.02 * rng.standard_normal((H, d))).astype(np.float32)
    return Inputs(wl, q, k, v, eta, wl.eta_const, w0, w1, w2, gamma, beta)


def upstream_grads(wl: Workload, seed: int):
    """Gradients of a scalar objective with respect to the forward's outputs, for
    backward tests: dZ ~ N(0,1) [B,H,N,d] and dW_end ~ N(0,1) [B,H,d,d], fp32,
    drawn from PCG64(seed) in that order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dz = rng.standard_normal((wl.B, wl.H, wl.N, wl.d)).astype(np.float32)
    dw = rng.standard_normal((wl.B, wl.H, wl.d, wl.d)).astype(np.float32)
    return dz, dw


def workload_inputs(index: int) -> Inputs:
    """Inputs of the index-th named workload with its documented seed."""
    return generate(WORKLOADS[index], SEED_BASE + index)


@dataclass(frozen=True)
class LayerWorkload:
    name: str
    kind: str            # inner model: "plain" | "ln"
    B: int
    N: int
    D: int
    H: int
    d: int
    b: int
    ln_eps: float = 1e-6
    description: str = ""


LAYER_SEED_BASE = 20261303

LAYER_WORKLOADS = [
    LayerWorkload("layer_ln_B8N2048_D768_H12_d64_b16", "ln", 8, 2048, 768, 12, 64, 16,
                  description="whole TTT layer around TTT-Linear+LN: bf16 x and projections, "
                              "B=8 N=2048 D=768 H=12 d=64 b=16, per-token eta"),
]


@dataclass
class LayerInputs:
    """Rounded whole-layer inputs; bf16 arrays hold bit patterns (uint16)."""
    wl: LayerWorkload
    x: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    w0: np.ndarray
    eta: np.ndarray
    gamma: Optional[np.ndarray]
    beta: Optional[np.ndarray]
    gamma_o: np.ndarray
    beta_o: np.ndarray

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if name in ("x", "wq", "wk", "wv", "wo"):
            return storage_to_f64(a, "bf16")
        return None if a is None else np.asarray(a, dtype=np.float64)


def generate_layer(wl: LayerWorkload, seed: int) -> LayerInputs:
    """Draw the inputs of a whole-layer workload from ``PCG64(seed)`` in the documented order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, N, D, H, d = wl.B, wl.N, wl.D, wl.H, wl.d
    HD = H * d
    bf = lambda a: _round_store(a, "bf16")
    x = bf(rng.standard_normal((B, N, D)))
    wq = bf(rng.standard_normal((HD, D)) / np.sqrt(D))
    wk = bf(rng.standard_normal((HD, D)) / np.sqrt(D))
    wv = bf(rng.standard_normal((HD, D)) / np.sqrt(D))
    wo = bf(rng.standard_normal((D, HD)) / np.sqrt(HD))
    w0 = (rng.standard_normal((B, H, d, d)) / np.sqrt(d)).astype(np.float32)
    u = rng.standard_normal((B, H, N))
    eta = (1.0 / (1.0 + np.exp(-u)) / d).astype(np.float32)
    gamma = beta = None
    if wl.kind == "ln":
        gamma = (1.0 + 0.02 * rng.standard_normal((H, d))).astype(np.float32)
        beta = (0.02 * rng.standard_normal((H, d))).astype(np.float32)
    gamma_o = (1.0 + 0.02 * rng.standard_normal((H, d))).astype(np.float32)
    beta_o = (0.02 * rng.standard_normal((H, d))).astype(np.float32)
    return LayerInputs(wl, x, wq, wk, wv, wo, w0, eta, gamma, beta, gamma_o, beta_o)


def layer_workload_inputs(index: int) -> LayerInputs:
    return generate_layer(LAYER_WORKLOADS[index], LAYER_SEED_BASE + index)


def layer_to_device(inp: LayerInputs, device="cuda"):
    """Device tensors of a whole-layer problem (bf16 arrays keep their bit patterns)."""
    import torch

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    def f32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    return dict(x=bf16(inp.x), wq=bf16(inp.wq), wk=bf16(inp.wk), wv=bf16(inp.wv), wo=bf16(inp.wo),
                w0=f32(inp.w0), eta=f32(inp.eta), gamma=f32(inp.gamma), beta=f32(inp.beta),
                gamma_o=f32(inp.gamma_o), beta_o=f32(inp.beta_o))


def to_device(inp: Inputs, device="cuda"):
    """Copy rounded inputs to device tensors (bf16 streams keep their bit patterns)."""
    import torch

    def stream(a):
        if inp.wl.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(a).to(device)

    def f32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    return dict(q=stream(inp.q), k=stream(inp.k), v=stream(inp.v), eta=f32(inp.eta),
                w0=f32(inp.w0), w1=f32(inp.w1), w2=f32(inp.w2), gamma=f32(inp.gamma),
                beta=f32(inp.beta))
