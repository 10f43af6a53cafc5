"""Thin Python binding of libttt.so (the C ABI in include/ttt.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs are allocated with torch, and the device pointers plus the
current HIP stream are handed to the C entry points, which run every step of
the computation in the library's HIP kernels. There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libttt.so")

TTT_OK, TTT_ERR_INVALID_ARGUMENT, TTT_ERR_UNSUPPORTED, TTT_ERR_WORKSPACE_TOO_SMALL, TTT_ERR_HIP = range(5)
TTT_DTYPE_F32, TTT_DTYPE_BF16 = 0, 1
TTT_LINEAR_PLAIN, TTT_LINEAR_LN = 0, 1
TTT_PATH_NONE, TTT_PATH_SMALL_B, TTT_PATH_LARGE_CHUNK = 0, 1, 2

KINDS = {"plain": TTT_LINEAR_PLAIN, "ln": TTT_LINEAR_LN}

_lib = None


class TTTError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libttt.so once and declare the C signatures. Raises if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m weights_ttt_layer_amd.build`")
    lib = ctypes.CDLL(path)
    vp, fp, i, f, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.ttt_linear_fwd.argtypes = [i, i, i, i, i, i, i, vp, vp, vp, fp, f, fp, fp, fp, f, fp, fp, vp,
                                   sz, vp]
    lib.ttt_linear_fwd.restype = i
    lib.ttt_linear_fwd_noalloc.argtypes = [i, i, i, i, i, i, i, vp, vp, vp, fp, f, fp, fp, fp, f, fp, fp, vp]
    lib.ttt_linear_fwd_noalloc.restype = i
    lib.ttt_linear_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.ttt_linear_fwd_workspace_bytes.restype = sz
    lib.ttt_linear_fwd_path.argtypes = [i, i, i, i]
    lib.ttt_linear_fwd_path.restype = i
    lib.ttt_mlp_fwd.argtypes = [i, i, i, i, i, i, i, vp, vp, vp, fp, f, fp, fp, fp, fp, f, fp, fp, fp,
                                vp, sz, vp]
    lib.ttt_mlp_fwd.restype = i
    lib.ttt_mlp_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.ttt_mlp_fwd_workspace_bytes.restype = sz
    lib.ttt_linear_fwd_block.argtypes = [i] + lib.ttt_linear_fwd.argtypes
    lib.ttt_linear_fwd_block.restype = i
    lib.ttt_linear_fwd_block_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
    lib.ttt_linear_fwd_block_workspace_bytes.restype = sz
    lib.ttt_linear_decode.argtypes = [i, i, i, i, i, vp, vp, vp, fp, f, fp, fp, fp, f, fp, vp]
    lib.ttt_linear_decode.restype = i
    lib.ttt_linear_bwd.argtypes = [i, i, i, i, i, i, i, vp, vp, vp, fp, f, fp, fp, fp, f, fp, fp, fp, fp, fp,
                                   fp, fp, fp, fp, vp, sz, vp]
    lib.ttt_linear_bwd.restype = i
    lib.ttt_linear_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.ttt_linear_bwd_workspace_bytes.restype = sz
    lib.ttt_layer_fwd.argtypes = [i, i, i, i, i, i, i, vp, vp, vp, vp, vp, fp, f, fp, fp, fp, fp, fp, f,
                                  fp, fp, vp, sz, vp]
    lib.ttt_layer_fwd.restype = i
    lib.ttt_layer_fwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.ttt_layer_fwd_workspace_bytes.restype = sz
    lib.ttt_status_string.argtypes = [i]
    lib.ttt_status_string.restype = ctypes.c_char_p
    lib.ttt_abi_version.argtypes = []
    lib.ttt_abi_version.restype = i
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ttt_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _qkv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TTT_DTYPE_BF16
    if t.dtype == torch.float32:
        return TTT_DTYPE_F32
    raise TypeError(f"Q/K/V must be bfloat16 or float32, got {t.dtype}")


def _on_device(t: torch.Tensor) -> bool:
    return t.is_cuda


def _check(t: torch.Tensor, name: str, shape, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not _on_device(t):
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def linear_path(kind: str, dtype: torch.dtype, d: int, b: int) -> int:
    return load_library().ttt_linear_fwd_path(KINDS[kind], _qkv_dtype(torch.empty(0, dtype=dtype)), d, b)


def linear_workspace_bytes(kind: str, dtype: torch.dtype, B: int, H: int, N: int, d: int, b: int) -> int:
    return int(load_library().ttt_linear_fwd_workspace_bytes(
        KINDS[kind], _qkv_dtype(torch.empty(0, dtype=dtype)), B, H, N, d, b))


APPLY = {"before": 0, "after": 1}


def _linear_call(entry: str, apply: Optional[int], q, k, v, w0, eta, b, kind, eta_const, ln_gamma,
                 ln_beta, ln_eps, z, w_end, workspace, stream, noalloc: bool = False):
    lib = load_library()
    if kind not in KINDS:
        raise ValueError(f"kind must be one of {sorted(KINDS)}")
    B, H, N, d = q.shape
    dt = _qkv_dtype(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm, (B, H, N, d), q.dtype)
    _check(w0, "w0", (B, H, d, d), torch.float32)
    if eta is not None:
        _check(eta, "eta", (B, H, N), torch.float32)
    if kind == "ln":
        if ln_gamma is None or ln_beta is None:
            raise ValueError("kind 'ln' needs ln_gamma and ln_beta")
        _check(ln_gamma, "ln_gamma", (H, d), torch.float32)
        _check(ln_beta, "ln_beta", (H, d), torch.float32)
    if z is None:
        z = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    else:
        _check(z, "z", (B, H, N, d), torch.float32)
    if w_end is None:
        w_end = torch.empty_like(w0)
    else:
        _check(w_end, "w_end", (B, H, d, d), torch.float32)
    args = (KINDS[kind], dt, B, H, N, d, int(b))
    if noalloc:
        st = lib.ttt_linear_fwd_noalloc(*args, _ptr(q), _ptr(k), _ptr(v), _ptr(eta), float(eta_const), _ptr(w0),
                                        _ptr(ln_gamma), _ptr(ln_beta), float(ln_eps), _ptr(z), _ptr(w_end),
                                        _stream_ptr(stream))
        if st != TTT_OK:
            raise TTTError(st, entry)
        return z, w_end
    if apply is None:
        need = int(lib.ttt_linear_fwd_workspace_bytes(*args))
    else:
        need = int(lib.ttt_linear_fwd_block_workspace_bytes(apply, *args))
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rest = (_ptr(q), _ptr(k), _ptr(v), _ptr(eta), float(eta_const), _ptr(w0), _ptr(ln_gamma),
            _ptr(ln_beta), float(ln_eps), _ptr(z), _ptr(w_end), _ptr(workspace), ws_bytes,
            _stream_ptr(stream))
    if apply is None:
        st = lib.ttt_linear_fwd(*args, *rest)
    else:
        st = lib.ttt_linear_fwd_block(apply, *args, *rest)
    if st != TTT_OK:
        raise TTTError(st, entry)
    return z, w_end


def linear_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w0: torch.Tensor,
               eta: Optional[torch.Tensor] = None, *, b: int, kind: str = "plain",
               eta_const: float = 0.0, ln_gamma: Optional[torch.Tensor] = None,
               ln_beta: Optional[torch.Tensor] = None, ln_eps: float = 1e-6,
               z: Optional[torch.Tensor] = None, w_end: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """TTT-Linear forward through ``ttt_linear_fwd``. Returns (Z, W_end).

    q, k, v: [B,H,N,d] bf16 or fp32; w0: [B,H,d,d] fp32; eta: [B,H,N] fp32 or
    None (then ``eta_const`` for every token); ln_gamma/ln_beta: [H,d] fp32 for
    kind "ln". ``w_end`` may be ``w0`` for an in-place state update.
    """
    return _linear_call("ttt_linear_fwd", None, q, k, v, w0, eta, b, kind, eta_const, ln_gamma,
                        ln_beta, ln_eps, z, w_end, workspace, stream)


def linear_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w0: torch.Tensor,
                       eta: Optional[torch.Tensor] = None, *, b: int, kind: str = "plain",
                       eta_const: float = 0.0, ln_gamma: Optional[torch.Tensor] = None,
                       ln_beta: Optional[torch.Tensor] = None, ln_eps: float = 1e-6,
                       z: Optional[torch.Tensor] = None, w_end: Optional[torch.Tensor] = None,
                       stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """``linear_fwd`` through ``ttt_linear_fwd_noalloc``: the large-chunk path
    uses the library's static device scratch instead of a workspace (outputs the
    caller does not pass are still allocated here by torch). Returns (Z, W_end)."""
    return _linear_call("ttt_linear_fwd_noalloc", None, q, k, v, w0, eta, b, kind, eta_const, ln_gamma,
                        ln_beta, ln_eps, z, w_end, None, stream, noalloc=True)


def linear_fwd_block(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w0: torch.Tensor,
                     eta: Optional[torch.Tensor] = None, *, b: int, apply: str = "before",
                     kind: str = "plain", eta_const: float = 0.0,
                     ln_gamma: Optional[torch.Tensor] = None, ln_beta: Optional[torch.Tensor] = None,
                     ln_eps: float = 1e-6, z: Optional[torch.Tensor] = None,
                     w_end: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Block-causal large-chunk forward through ``ttt_linear_fwd_block``: every
    output of chunk c uses W_c (apply="before") or W_{c+1} (apply="after").
    Arguments as for ``linear_fwd``. Returns (Z, W_end)."""
    if apply not in APPLY:
        raise ValueError(f"apply must be one of {sorted(APPLY)}")
    return _linear_call("ttt_linear_fwd_block", APPLY[apply], q, k, v, w0, eta, b, kind, eta_const,
                        ln_gamma, ln_beta, ln_eps, z, w_end, workspace, stream)


def linear_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w: torch.Tensor,
                  eta: Optional[torch.Tensor] = None, *, kind: str = "plain", eta_const: float = 0.0,
                  ln_gamma: Optional[torch.Tensor] = None, ln_beta: Optional[torch.Tensor] = None,
                  ln_eps: float = 1e-6, z: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode token per (sequence, head) through ``ttt_linear_decode``.

    q, k, v: [B,H,d]; w: [B,H,d,d] fp32, updated in place; eta: [B,H] fp32 or
    None. Returns z [B,H,d] fp32."""
    lib = load_library()
    if kind not in KINDS:
        raise ValueError(f"kind must be one of {sorted(KINDS)}")
    B, H, d = q.shape
    dt = _qkv_dtype(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm, (B, H, d), q.dtype)
    _check(w, "w", (B, H, d, d), torch.float32)
    if eta is not None:
        _check(eta, "eta", (B, H), torch.float32)
    if kind == "ln":
        if ln_gamma is None or ln_beta is None:
            raise ValueError("kind 'ln' needs ln_gamma and ln_beta")
        _check(ln_gamma, "ln_gamma", (H, d), torch.float32)
        _check(ln_beta, "ln_beta", (H, d), torch.float32)
    if z is None:
        z = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    else:
        _check(z, "z", (B, H, d), torch.float32)
    st = lib.ttt_linear_decode(KINDS[kind], dt, B, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                               float(eta_const), _ptr(w), _ptr(ln_gamma), _ptr(ln_beta), float(ln_eps),
                               _ptr(z), _stream_ptr(stream))
    if st != TTT_OK:
        raise TTTError(st, "ttt_linear_decode")
    return z


def mlp_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor,
            eta: Optional[torch.Tensor] = None, *, b: int, ln_gamma: torch.Tensor,
            ln_beta: torch.Tensor, eta_const: float = 0.0, ln_eps: float = 1e-6,
            z: Optional[torch.Tensor] = None, w1_end: Optional[torch.Tensor] = None,
            w2_end: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None
            ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """TTT-MLP forward through ``ttt_mlp_fwd``. Returns (Z, W1_end, W2_end). The
    workspace (needed beyond d = 64 with b <= 16) is allocated here unless given."""
    lib = load_library()
    B, H, N, d = q.shape
    hid = w1.shape[-1]
    dt = _qkv_dtype(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm, (B, H, N, d), q.dtype)
    _check(w1, "w1", (B, H, d, hid), torch.float32)
    _check(w2, "w2", (B, H, hid, d), torch.float32)
    if eta is not None:
        _check(eta, "eta", (B, H, N), torch.float32)
    _check(ln_gamma, "ln_gamma", (H, d), torch.float32)
    _check(ln_beta, "ln_beta", (H, d), torch.float32)
    if z is None:
        z = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    else:
        _check(z, "z", (B, H, N, d), torch.float32)
    if w1_end is None:
        w1_end = torch.empty_like(w1)
    else:
        _check(w1_end, "w1_end", (B, H, d, hid), torch.float32)
    if w2_end is None:
        w2_end = torch.empty_like(w2)
    else:
        _check(w2_end, "w2_end", (B, H, hid, d), torch.float32)
    need = int(lib.ttt_mlp_fwd_workspace_bytes(dt, B, H, N, d, hid, int(b)))
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ttt_mlp_fwd(dt, B, H, N, d, hid, int(b), _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                         float(eta_const), _ptr(w1), _ptr(w2), _ptr(ln_gamma), _ptr(ln_beta),
                         float(ln_eps), _ptr(z), _ptr(w1_end), _ptr(w2_end), _ptr(workspace), ws_bytes,
                         _stream_ptr(stream))
    if st != TTT_OK:
        raise TTTError(st, "ttt_mlp_fwd")
    return z, w1_end, w2_end


def layer_workspace_bytes(B: int, N: int, H: int, d: int) -> int:
    return int(load_library().ttt_layer_fwd_workspace_bytes(B, N, H, d))


def layer_fwd(x: torch.Tensor, wq: torch.Tensor, wk: torch.Tensor, wv: torch.Tensor,
              wo: torch.Tensor, w0: torch.Tensor, out_gamma: torch.Tensor, out_beta: torch.Tensor,
              eta: Optional[torch.Tensor] = None, *, H: int, b: int, kind: str = "plain",
              eta_const: float = 0.0, ln_gamma: Optional[torch.Tensor] = None,
              ln_beta: Optional[torch.Tensor] = None, ln_eps: float = 1e-6,
              y: Optional[torch.Tensor] = None, w_end: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None
              ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """The whole layer through ``ttt_layer_fwd``. Returns (y, W_end, workspace).

    x: [B,N,D] bf16; wq, wk, wv: [H*d, D] bf16; wo: [D, H*d] bf16; w0: [B,H,d,d]
    fp32; out_gamma/out_beta (and ln_gamma/ln_beta for kind "ln"): [H,d] fp32;
    eta: [B,H,N] fp32 or None. The returned workspace holds the fp32 Q, K, V, Z
    arrays ([B,H,N,d] each, see ``layer_parts``)."""
    lib = load_library()
    if kind not in KINDS:
        raise ValueError(f"kind must be one of {sorted(KINDS)}")
    B, N, D = x.shape
    HD = wq.shape[0]
    if HD % H != 0:
        raise ValueError(f"projection width {HD} is not a multiple of H={H}")
    d = HD // H
    _check(x, "x", (B, N, D), torch.bfloat16)
    for t, nm in ((wq, "wq"), (wk, "wk"), (wv, "wv")):
        _check(t, nm, (HD, D), torch.bfloat16)
    _check(wo, "wo", (D, HD), torch.bfloat16)
    _check(w0, "w0", (B, H, d, d), torch.float32)
    _check(out_gamma, "out_gamma", (H, d), torch.float32)
    _check(out_beta, "out_beta", (H, d), torch.float32)
    if eta is not None:
        _check(eta, "eta", (B, H, N), torch.float32)
    if kind == "ln":
        if ln_gamma is None or ln_beta is None:
            raise ValueError("kind 'ln' needs ln_gamma and ln_beta")
        _check(ln_gamma, "ln_gamma", (H, d), torch.float32)
        _check(ln_beta, "ln_beta", (H, d), torch.float32)
    if y is None:
        y = torch.empty((B, N, D), dtype=torch.float32, device=x.device)
    else:
        _check(y, "y", (B, N, D), torch.float32)
    if w_end is None:
        w_end = torch.empty_like(w0)
    else:
        _check(w_end, "w_end", (B, H, d, d), torch.float32)
    need = int(lib.ttt_layer_fwd_workspace_bytes(B, N, H, d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.ttt_layer_fwd(KINDS[kind], B, N, D, H, d, int(b), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv),
                           _ptr(wo), _ptr(eta), float(eta_const), _ptr(w0), _ptr(ln_gamma),
                           _ptr(ln_beta), _ptr(out_gamma), _ptr(out_beta), float(ln_eps), _ptr(y),
                           _ptr(w_end), _ptr(workspace), ws_bytes, _stream_ptr(stream))
    if st != TTT_OK:
        raise TTTError(st, "ttt_layer_fwd")
    return y, w_end, workspace


def layer_parts(workspace: torch.Tensor, B: int, N: int, H: int, d: int) -> dict:
    """The Q, K, V, Z arrays a ``layer_fwd`` call left in its workspace, fp32
    [B, H, N, d]. Q, K, V are stored as two bf16 planes each (hi, then lo) and
    returned as their sum; Z is a view of the fp32 array."""
    region = int(load_library().ttt_layer_fwd_workspace_bytes(B, N, H, d)) // 5
    n = B * H * N * d
    out = {}
    for i, name in enumerate("QKV"):
        planes = workspace[i * region:i * region + 4 * n].view(torch.bfloat16)
        out[name] = (planes[:n].float() + planes[n:].float()).view(B, H, N, d)
    out["Z"] = workspace[3 * region:3 * region + 4 * n].view(torch.float32).view(B, H, N, d)
    return out


def linear_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w0: torch.Tensor, dz: torch.Tensor,
               eta: Optional[torch.Tensor] = None, *, b: int, kind: str = "plain", eta_const: float = 0.0,
               dw_end: Optional[torch.Tensor] = None, ln_gamma: Optional[torch.Tensor] = None,
               ln_beta: Optional[torch.Tensor] = None, ln_eps: float = 1e-6,
               workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Backward of ``linear_fwd`` through ``ttt_linear_bwd``. Returns a dict of
    dQ, dK, dV ([B,H,N,d]), deta ([B,H,N]), dW0 ([B,H,d,d]) and, for kind "ln",
    dgamma, dbeta ([H,d]); all fp32."""
    lib = load_library()
    if kind not in KINDS:
        raise ValueError(f"kind must be one of {sorted(KINDS)}")
    B, H, N, d = q.shape
    dt = _qkv_dtype(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm, (B, H, N, d), q.dtype)
    _check(w0, "w0", (B, H, d, d), torch.float32)
    _check(dz, "dz", (B, H, N, d), torch.float32)
    if dw_end is not None:
        _check(dw_end, "dw_end", (B, H, d, d), torch.float32)
    if eta is not None:
        _check(eta, "eta", (B, H, N), torch.float32)
    if kind == "ln":
        if ln_gamma is None or ln_beta is None:
            raise ValueError("kind 'ln' needs ln_gamma and ln_beta")
        _check(ln_gamma, "ln_gamma", (H, d), torch.float32)
        _check(ln_beta, "ln_beta", (H, d), torch.float32)
    dev = q.device
    out = {name: torch.empty((B, H, N, d), dtype=torch.float32, device=dev) for name in ("dQ", "dK", "dV")}
    out["deta"] = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    out["dW0"] = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    out["dgamma"] = torch.empty((H, d), dtype=torch.float32, device=dev) if kind == "ln" else None
    out["dbeta"] = torch.empty((H, d), dtype=torch.float32, device=dev) if kind == "ln" else None
    need = int(lib.ttt_linear_bwd_workspace_bytes(KINDS[kind], dt, B, H, N, d, int(b)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.ttt_linear_bwd(KINDS[kind], dt, B, H, N, d, int(b), _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                            float(eta_const), _ptr(w0), _ptr(ln_gamma), _ptr(ln_beta), float(ln_eps), _ptr(dz),
                            _ptr(dw_end), _ptr(out["dQ"]), _ptr(out["dK"]), _ptr(out["dV"]), _ptr(out["deta"]),
                            _ptr(out["dW0"]), _ptr(out["dgamma"]), _ptr(out["dbeta"]), _ptr(workspace), ws_bytes,
                            _stream_ptr(stream))
    if st != TTT_OK:
        raise TTTError(st, "ttt_linear_bwd")
    return out


# ---------------------------------------------------------------------------
# Calibration library (include/ttt_peak.h): practical device peaks for the
# measurements; not used by any forward or backward call.
# ---------------------------------------------------------------------------
PEAK_LIB_PATH = os.path.join(_HERE, "libttt_peak.so")
_peak_lib = None


def load_peak_library(path: str = PEAK_LIB_PATH) -> ctypes.CDLL:
    """Load libttt_peak.so once and declare its C signatures."""
    global _peak_lib
    if _peak_lib is not None:
        return _peak_lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m weights_ttt_layer_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, sz, ip = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int)
    lib.ttt_peak_device_info.argtypes = [i, ip, ip, ip]
    lib.ttt_peak_device_info.restype = i
    lib.ttt_peak_copy.argtypes = [vp, vp, sz, vp]
    lib.ttt_peak_copy.restype = i
    lib.ttt_peak_mfma.argtypes = [vp, i, i, vp]
    lib.ttt_peak_mfma.restype = i
    lib.ttt_peak_mfma_flops.argtypes = [i, i]
    lib.ttt_peak_mfma_flops.restype = ctypes.c_double
    _peak_lib = lib
    return lib


def peak_device_info(device: int = 0) -> dict:
    """Compute units, shader clock (kHz) and wavefront width of a device."""
    lib = load_peak_library()
    cu, clk, wf = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    st = lib.ttt_peak_device_info(int(device), ctypes.byref(cu), ctypes.byref(clk), ctypes.byref(wf))
    if st != TTT_OK:
        raise TTTError(st, "ttt_peak_device_info")
    return {"compute_units": cu.value, "clock_khz": clk.value, "wavefront_size": wf.value}


def peak_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """dst <- src through the calibration copy kernel (same byte size, 16-byte multiple)."""
    lib = load_peak_library()
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("peak_copy needs contiguous tensors of the same byte size")
    st = lib.ttt_peak_copy(_ptr(src), _ptr(dst), nbytes, _stream_ptr(stream))
    if st != TTT_OK:
        raise TTTError(st, "ttt_peak_copy")


def peak_mfma(out: torch.Tensor, blocks: int, iters: int, stream=None) -> float:
    """Run the MFMA loop (out: >= blocks * 256 fp32); returns the flops it performs."""
    lib = load_peak_library()
    if out.dtype != torch.float32 or out.numel() < blocks * 256 or not out.is_contiguous():
        raise ValueError("peak_mfma needs a contiguous fp32 tensor of at least blocks * 256 elements")
    st = lib.ttt_peak_mfma(_ptr(out), int(blocks), int(iters), _stream_ptr(stream))
    if st != TTT_OK:
        raise TTTError(st, "ttt_peak_mfma")
    return float(lib.ttt_peak_mfma_flops(int(blocks), int(iters)))
