"""fp64 CPU oracle for the TTT-layer forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library never does, and the
two share no code: this wrapper only marshals numpy arrays into the plain C
routines of ``ttt_oracle.c`` (see that file's header for what is computed and
which passage of the pages each part follows).

Every array is converted to contiguous float64 before the call; callers pass
the exact values the GPU receives (bf16/fp32 inputs upcast), so input rounding
is not part of any parity error.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ttt_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libttt_oracle.so")

ONLINE, MINIBATCH, DUAL, BLOCK_BEFORE, BLOCK_AFTER = 0, 1, 2, 3, 4
PLAIN, LN = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile ttt_oracle.c with gcc (fp64, IEEE, OpenMP). Returns the .so path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(ctypes.c_double)
    i, d = ctypes.c_int, ctypes.c_double
    lib.ttt_oracle_linear.argtypes = [i, i, i, i, i, i, i, P, P, P, P, P, P, P, d, P, P, i]
    lib.ttt_oracle_linear.restype = i
    lib.ttt_oracle_mlp.argtypes = [i, i, i, i, i, i, i, P, P, P, P, P, P, P, P, d, P, P, P, i]
    lib.ttt_oracle_mlp.restype = i
    lib.ttt_oracle_linear_loss.argtypes = [i, i, P, P, P, P, P, d]
    lib.ttt_oracle_linear_loss.restype = d
    lib.ttt_oracle_linear_grad.argtypes = [i, i, P, P, P, P, P, d, P]
    lib.ttt_oracle_linear_grad.restype = None
    lib.ttt_oracle_mlp_loss.argtypes = [i, i, P, P, P, P, P, P, d]
    lib.ttt_oracle_mlp_loss.restype = d
    lib.ttt_oracle_mlp_grad.argtypes = [i, i, P, P, P, P, P, P, d, P, P]
    lib.ttt_oracle_mlp_grad.restype = None
    lib.ttt_oracle_linear_bwd.argtypes = [i, i, i, i, i, i, P, P, P, P, P, P, P, d, P, P, P, P, P, P, P,
                                          P, P, i]
    lib.ttt_oracle_linear_bwd.restype = i
    lib.ttt_oracle_gelu.argtypes = [d]
    lib.ttt_oracle_gelu.restype = d
    lib.ttt_oracle_gelu_prime.argtypes = [d]
    lib.ttt_oracle_gelu_prime.restype = d
    _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _eta_array(eta, B, H, N):
    if np.isscalar(eta) or np.ndim(eta) == 0:
        return np.full((B, H, N), float(eta), dtype=np.float64)
    return _f64(eta).reshape(B, H, N)


def _default_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def linear(mode, kind, Q, K, V, eta, W0, b, gamma=None, beta=None, eps=1e-6, nthreads=None):
    """TTT-Linear (kind PLAIN or LN) over [B,H,N,d] inputs. Returns (Z, W_end) fp64.

    ``eta`` is a scalar or a [B,H,N] array (step size of each source token).
    ``gamma``/``beta`` are [H,d] for kind LN.
    """
    lib = _load()
    Q, K, V, W0 = _f64(Q), _f64(K), _f64(V), _f64(W0)
    B, H, N, d = Q.shape
    assert K.shape == Q.shape and V.shape == Q.shape and W0.shape == (B, H, d, d)
    e = _eta_array(eta, B, H, N)
    g = _f64(gamma).reshape(H, d) if kind == LN else None
    bt = _f64(beta).reshape(H, d) if kind == LN else None
    Z = np.zeros((B, H, N, d))
    We = np.zeros((B, H, d, d))
    rc = lib.ttt_oracle_linear(mode, kind, B, H, N, d, int(b), _ptr(Q), _ptr(K), _ptr(V), _ptr(e),
                               _ptr(W0), _ptr(g), _ptr(bt), float(eps), _ptr(Z), _ptr(We),
                               nthreads or _default_threads())
    if rc != 0:
        raise ValueError("ttt_oracle_linear rejected its arguments")
    return Z, We


def linear_bwd(kind, Q, K, V, eta, W0, b, dZ, dW_end=None, gamma=None, beta=None, eps=1e-6,
               nthreads=None):
    """Gradients of TTT-Linear (kind PLAIN or LN, the mini-batch dual form) with
    respect to all inputs, given dZ [B,H,N,d] and dW_end [B,H,d,d] (None = 0).
    Returns dict(dQ, dK, dV, deta [B,H,N], dW0, dgamma, dbeta [H,d] or None)."""
    lib = _load()
    Q, K, V, W0, dZ = _f64(Q), _f64(K), _f64(V), _f64(W0), _f64(dZ)
    B, H, N, d = Q.shape
    e = _eta_array(eta, B, H, N)
    g = _f64(gamma).reshape(H, d) if kind == LN else None
    bt = _f64(beta).reshape(H, d) if kind == LN else None
    dWe = None if dW_end is None else _f64(dW_end)
    out = {k: np.zeros((B, H, N, d)) for k in ("dQ", "dK", "dV")}
    out["deta"] = np.zeros((B, H, N))
    out["dW0"] = np.zeros((B, H, d, d))
    out["dgamma"] = np.zeros((H, d)) if kind == LN else None
    out["dbeta"] = np.zeros((H, d)) if kind == LN else None
    rc = lib.ttt_oracle_linear_bwd(kind, B, H, N, d, int(b), _ptr(Q), _ptr(K), _ptr(V), _ptr(e), _ptr(W0),
                                   _ptr(g), _ptr(bt), float(eps), _ptr(dZ), _ptr(dWe), _ptr(out["dQ"]),
                                   _ptr(out["dK"]), _ptr(out["dV"]), _ptr(out["deta"]), _ptr(out["dW0"]),
                                   _ptr(out["dgamma"]), _ptr(out["dbeta"]), nthreads or _default_threads())
    if rc != 0:
        raise ValueError("ttt_oracle_linear_bwd rejected its arguments")
    return out


def mlp(mode, Q, K, V, eta, W1, W2, b, gamma, beta, eps=1e-6, nthreads=None):
    """TTT-MLP f(x) = x + LN(GELU(x W1) W2). Returns (Z, W1_end, W2_end) fp64."""
    lib = _load()
    Q, K, V, W1, W2 = _f64(Q), _f64(K), _f64(V), _f64(W1), _f64(W2)
    B, H, N, d = Q.shape
    hid = W1.shape[-1]
    assert W1.shape == (B, H, d, hid) and W2.shape == (B, H, hid, d)
    e = _eta_array(eta, B, H, N)
    g = _f64(gamma).reshape(H, d)
    bt = _f64(beta).reshape(H, d)
    Z = np.zeros((B, H, N, d))
    W1e = np.zeros_like(W1)
    W2e = np.zeros_like(W2)
    rc = lib.ttt_oracle_mlp(mode, B, H, N, d, hid, int(b), _ptr(Q), _ptr(K), _ptr(V), _ptr(e),
                            _ptr(W1), _ptr(W2), _ptr(g), _ptr(bt), float(eps), _ptr(Z), _ptr(W1e),
                            _ptr(W2e), nthreads or _default_threads())
    if rc != 0:
        raise ValueError("ttt_oracle_mlp rejected its arguments")
    return Z, W1e, W2e


def linear_loss(kind, W, k, v, gamma=None, beta=None, eps=1e-6):
    """Per-token loss ||f(k;W) - v||^2 for one token."""
    lib = _load()
    W, k, v = _f64(W), _f64(k), _f64(v)
    d = k.shape[0]
    g = _f64(gamma) if gamma is not None else None
    bt = _f64(beta) if beta is not None else None
    return lib.ttt_oracle_linear_loss(kind, d, _ptr(W), _ptr(k), _ptr(v), _ptr(g), _ptr(bt),
                                      float(eps))


def linear_grad(kind, W, k, v, gamma=None, beta=None, eps=1e-6):
    """Analytic gradient d loss / d W for one token, [d,d]."""
    lib = _load()
    W, k, v = _f64(W), _f64(k), _f64(v)
    d = k.shape[0]
    g = _f64(gamma) if gamma is not None else None
    bt = _f64(beta) if beta is not None else None
    dW = np.zeros((d, d))
    lib.ttt_oracle_linear_grad(kind, d, _ptr(W), _ptr(k), _ptr(v), _ptr(g), _ptr(bt), float(eps),
                               _ptr(dW))
    return dW


def mlp_loss(W1, W2, k, v, gamma, beta, eps=1e-6):
    lib = _load()
    W1, W2, k, v, g, bt = map(_f64, (W1, W2, k, v, gamma, beta))
    d, hid = W1.shape
    return lib.ttt_oracle_mlp_loss(d, hid, _ptr(W1), _ptr(W2), _ptr(k), _ptr(v), _ptr(g), _ptr(bt),
                                   float(eps))


def mlp_grad(W1, W2, k, v, gamma, beta, eps=1e-6):
    """Analytic gradients (dW1 [d,hid], dW2 [hid,d]) for one token."""
    lib = _load()
    W1, W2, k, v, g, bt = map(_f64, (W1, W2, k, v, gamma, beta))
    d, hid = W1.shape
    dW1 = np.zeros((d, hid))
    dW2 = np.zeros((hid, d))
    lib.ttt_oracle_mlp_grad(d, hid, _ptr(W1), _ptr(W2), _ptr(k), _ptr(v), _ptr(g), _ptr(bt),
                            float(eps), _ptr(dW1), _ptr(dW2))
    return dW1, dW2


def gelu(a: float) -> float:
    return _load().ttt_oracle_gelu(float(a))


def gelu_prime(a: float) -> float:
    return _load().ttt_oracle_gelu_prime(float(a))


def layer_norm(x, gamma, beta, eps):
    """LayerNorm over the last axis: biased variance, eps inside the square root."""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    return xc / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


def layer(kind, x, Wq, Wk, Wv, Wo, eta, W0, b, H, gamma=None, beta=None, gamma_o=None,
          beta_o=None, eps=1e-6, mode=DUAL, nthreads=None):
    """The whole TTT layer around the inner model (TTT-Linear, kind PLAIN or LN).

    Page "Test-Time Training: Linear Complexity Beyond Attention":
      * section "1. The Self-Supervised Inner-Loop Task": each token x_t (a model
        vector of width D) is projected to query, key and value, q_t = W_Q x_t,
        k_t = W_K x_t, v_t = W_V x_t. The projections are [H*d, D] matrices
        (output index first); the H*d outputs are H heads of width d, head h
        taking outputs h*d .. h*d + d - 1.
      * the same page's layer code normalises each key to unit L2 length
        before the inner loop (a zero key stays zero).
      * the inner model runs per (sequence, head) exactly as ``linear``.
      * section "3. Forward Evaluation and Output Projection": the output is
        y_t = W_O (LayerNorm(z_t) + q_t), the LayerNorm taken per head over the
        head's d entries with a per-head affine (gamma_o, beta_o of shape
        [H, d]); W_O is [D, H*d].

    ``x`` is [B, N, D]. Returns (y [B,N,D], W_end [B,H,d,d], parts) in fp64 where
    ``parts`` holds the intermediate Q, K (normalised), V and Z, each [B,H,N,d].
    """
    x = _f64(x)
    Bn, N, D = x.shape
    Wq, Wk, Wv, Wo = _f64(Wq), _f64(Wk), _f64(Wv), _f64(Wo)
    HD = Wq.shape[0]
    assert HD % H == 0 and Wq.shape == (HD, D) and Wk.shape == (HD, D) and Wv.shape == (HD, D)
    assert Wo.shape == (D, HD)
    d = HD // H

    def heads(P):                 # [B, N, H*d] -> [B, H, N, d]
        return np.ascontiguousarray(P.reshape(Bn, N, H, d).transpose(0, 2, 1, 3))

    Q = heads(x @ Wq.T)
    K = heads(x @ Wk.T)
    V = heads(x @ Wv.T)
    nrm = np.sqrt(np.sum(K * K, axis=-1, keepdims=True))
    K = K / np.where(nrm > 0, nrm, 1.0)
    Z, We = linear(mode, kind, Q, K, V, eta, W0, b, gamma, beta, eps, nthreads)
    go = _f64(gamma_o).reshape(H, 1, d)
    bo = _f64(beta_o).reshape(H, 1, d)
    A = layer_norm(Z, go, bo, eps) + Q                   # [B, H, N, d]
    y = A.transpose(0, 2, 1, 3).reshape(Bn, N, HD) @ Wo.T
    return y, We, dict(Q=Q, K=K, V=V, Z=Z)
