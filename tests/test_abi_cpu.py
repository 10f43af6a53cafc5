"""C-ABI contract tests that need no GPU: the library loads, exports every
symbol include/ttt.h declares, and rejects bad arguments on the host before any
HIP call (so nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt.h")

from weights_ttt_layer_amd import binding  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "ttt_linear_fwd" in names and "ttt_mlp_fwd" in names
    for n in names:
        assert hasattr(lib, n), f"libttt.so does not export {n}"


def test_version_and_status_strings(lib):
    assert lib.ttt_abi_version() == 2
    for s in range(5):
        assert binding.status_string(s).startswith("TTT_")
    assert binding.status_string(99) == "unknown ttt_status"


def test_path_selection(lib):
    P = lib.ttt_linear_fwd_path
    assert P(0, 0, 64, 16) == binding.TTT_PATH_SMALL_B
    assert P(1, 1, 64, 1) == binding.TTT_PATH_SMALL_B
    assert P(1, 1, 64, 17) == binding.TTT_PATH_SMALL_B
    assert P(0, 0, 64, 64) == binding.TTT_PATH_SMALL_B
    assert P(1, 0, 128, 1) == binding.TTT_PATH_SMALL_B
    assert P(1, 1, 128, 64) == binding.TTT_PATH_SMALL_B
    assert P(1, 1, 64, 65) == binding.TTT_PATH_NONE
    assert P(0, 1, 128, 2048) == binding.TTT_PATH_LARGE_CHUNK
    assert P(1, 1, 128, 2048) == binding.TTT_PATH_NONE       # LN has no large-chunk path
    assert P(1, 0, 64, 65) == binding.TTT_PATH_NONE
    assert P(0, 1, 128, 2000) == binding.TTT_PATH_LARGE_CHUNK  # any b > 64 for plain f
    assert P(0, 0, 64, 256) == binding.TTT_PATH_LARGE_CHUNK
    assert P(0, 1, 64, 65) == binding.TTT_PATH_LARGE_CHUNK
    assert P(0, 1, 32, 16) == binding.TTT_PATH_NONE
    assert P(5, 1, 64, 16) == binding.TTT_PATH_NONE


def test_workspace_sizes(lib):
    W = lib.ttt_linear_fwd_workspace_bytes
    assert W(0, 1, 8, 12, 2048, 64, 16) == 0          # small-b path needs none
    assert W(0, 1, 1, 16, 32768, 128, 2048) > 0
    assert W(0, 1, 0, 16, 32768, 128, 2048) == 0      # invalid sizes
    # combinations outside the chunk-parallel kernels need none
    assert W(0, 0, 1, 16, 32768, 128, 2048) == 0      # fp32 streams
    assert W(0, 1, 1, 1, 1000, 64, 256) == 0          # d = 64, ragged N
    assert W(0, 1, 1, 1, 1000, 128, 256) == 0         # N not a multiple of 128


# Fake, never-dereferenced device addresses: every call below must be rejected
# by host-side validation before anything is launched.
A = 1 << 40


def addr(i, size=1 << 30):
    return ctypes.c_void_p(A + i * size)


def lin_call(lib, kind=0, dt=1, B=1, H=1, N=64, d=64, b=16, Q=0, K=1, V=2, eta=None, W0=3,
             gam=4, bet=5, eps=1e-6, Z=6, We=7, ws=None, wsb=0):
    p = lambda i: None if i is None else (i if isinstance(i, ctypes.c_void_p) else addr(i))
    return lib.ttt_linear_fwd(kind, dt, B, H, N, d, b, p(Q), p(K), p(V), p(eta), 0.1, p(W0), p(gam),
                              p(bet), eps, p(Z), p(We), p(ws), wsb, None)


def test_rejects_invalid_arguments(lib):
    E = binding.TTT_ERR_INVALID_ARGUMENT
    assert lin_call(lib, kind=7) == E
    assert lin_call(lib, dt=3) == E
    assert lin_call(lib, B=0) == E
    assert lin_call(lib, N=0) == E
    assert lin_call(lib, b=0) == E
    assert lin_call(lib, Q=None) == E
    assert lin_call(lib, Z=None) == E
    assert lin_call(lib, We=None) == E
    assert lin_call(lib, kind=1, gam=None) == E
    assert lin_call(lib, kind=1, eps=-1.0) == E
    assert lin_call(lib, kind=1, eps=float("nan")) == E
    # misaligned token stream
    assert lin_call(lib, Q=ctypes.c_void_p(A + 2)) == E
    # Z overlapping an input
    assert lin_call(lib, Z=ctypes.c_void_p(A + 8)) == E
    # W_end partially overlapping W0 (equal is allowed, see below)
    assert lin_call(lib, We=ctypes.c_void_p(A + 3 * (1 << 30) + 64)) == E
    # Z and per-token eta are accessed with 16-byte vectors
    assert lin_call(lib, Z=ctypes.c_void_p(A + 6 * (1 << 30) + 4)) == E
    assert lin_call(lib, eta=ctypes.c_void_p(A + 8 * (1 << 30) + 4)) == E
    assert lin_call(lib, eta=ctypes.c_void_p(A + 8 * (1 << 30) + 16)) != E


def test_rejects_unsupported(lib):
    U = binding.TTT_ERR_UNSUPPORTED
    assert lin_call(lib, d=32) == U
    assert lin_call(lib, kind=1, b=65) == U
    assert lin_call(lib, kind=1, d=128, b=100) == U
    assert lin_call(lib, kind=1, d=128, b=2048) == U
    assert lin_call(lib, d=96, b=100) == U


def test_large_chunk_workspace_checked_before_launch(lib):
    rc = lin_call(lib, B=1, H=16, N=32768, d=128, b=2048, ws=None, wsb=0)
    assert rc == binding.TTT_ERR_WORKSPACE_TOO_SMALL


def test_large_chunk_workspace_must_not_overlap_eta(lib):
    # the large path writes its workspace while other workgroups still read eta
    need = lib.ttt_linear_fwd_workspace_bytes(0, 1, 1, 16, 32768, 128, 2048)
    assert need > 0
    rc = lin_call(lib, B=1, H=16, N=32768, d=128, b=2048, eta=ctypes.c_void_p(A + 9 * (1 << 30) + 256),
                  ws=9, wsb=need)
    assert rc == binding.TTT_ERR_INVALID_ARGUMENT
    rc = lin_call(lib, B=1, H=16, N=32768, d=128, b=2048, eta=8, ws=9, wsb=need)
    assert rc != binding.TTT_ERR_INVALID_ARGUMENT


def test_binding_checks_mlp_outputs_before_launch(monkeypatch):
    """mlp_fwd validates caller-supplied outputs (shape, dtype, contiguity) before
    the library is called: a wrong-shape z must raise, not reach the kernel."""
    import torch

    class NoLaunch:
        def __getattr__(self, name):
            raise AssertionError(f"{name} called despite an invalid output")

    monkeypatch.setattr(binding, "load_library", lambda *a, **k: NoLaunch())
    monkeypatch.setattr(binding, "_on_device", lambda t: True)
    B, H, N, d, hid = 1, 2, 8, 64, 256
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    w1 = torch.zeros((B, H, d, hid))
    w2 = torch.zeros((B, H, hid, d))
    g = torch.ones((H, d))
    kw = dict(b=4, ln_gamma=g, ln_beta=g)
    with pytest.raises(ValueError, match="z has shape"):
        binding.mlp_fwd(q, q, q, w1, w2, z=torch.zeros((B, H, N, d + 1)), **kw)
    with pytest.raises(TypeError, match="w1_end must be"):
        binding.mlp_fwd(q, q, q, w1, w2, w1_end=torch.zeros((B, H, d, hid), dtype=torch.float64), **kw)
    with pytest.raises(ValueError, match="w2_end must be contiguous"):
        binding.mlp_fwd(q, q, q, w1, w2, w2_end=torch.zeros((B, H, d, hid)).transpose(2, 3), **kw)


def test_mlp_rejections(lib):
    p = addr
    f = lib.ttt_mlp_fwd
    E, U = binding.TTT_ERR_INVALID_ARGUMENT, binding.TTT_ERR_UNSUPPORTED
    args = lambda **kw: dict(dict(dt=1, B=1, H=1, N=64, d=64, hid=256, b=16), **kw)

    def call(**kw):
        a = args(**kw)
        return f(a["dt"], a["B"], a["H"], a["N"], a["d"], a["hid"], a["b"], p(0), p(1), p(2), None,
                 0.1, a.get("W1", p(3)), p(4), a.get("gam", p(5)), p(6), 1e-6, p(7), p(8), p(9),
                 a.get("ws"), a.get("wsb", 0), None)
    W = lib.ttt_mlp_fwd_workspace_bytes
    assert call(dt=5) == E
    assert call(hid=0) == E
    assert call(gam=None) == E
    assert call(W1=None) == E
    assert call(d=32, hid=128) == U
    assert call(hid=128) == U
    assert call(b=65) == U
    assert W(1, 1, 1, 64, 64, 256, 16) == 0                # on-chip state
    need = W(1, 1, 1, 64, 64, 256, 32)
    assert need > 0 and W(1, 1, 1, 64, 128, 512, 16) > 0
    assert call(b=32) == binding.TTT_ERR_WORKSPACE_TOO_SMALL
    assert call(b=32, ws=p(10), wsb=need - 1) == binding.TTT_ERR_WORKSPACE_TOO_SMALL
    assert call(b=32, ws=ctypes.c_void_p(A + 10 * (1 << 30) + 16), wsb=need) == E   # misaligned
    assert call(b=32, ws=ctypes.c_void_p(A + 9 * (1 << 30) - 256), wsb=need) == E   # overlaps W2_end
    assert call(d=128, hid=512, b=16) == binding.TTT_ERR_WORKSPACE_TOO_SMALL


def block_call(lib, apply=0, kind=0, dt=1, B=1, H=16, N=32768, d=128, b=2048, ws=None, wsb=0, Z=6):
    return lib.ttt_linear_fwd_block(apply, kind, dt, B, H, N, d, b, addr(0), addr(1), addr(2), None, 0.1,
                                    addr(3), addr(4), addr(5), 1e-6, None if Z is None else addr(Z), addr(7),
                                    None if ws is None else addr(ws), wsb, None)


def test_block_rejections(lib):
    E, U = binding.TTT_ERR_INVALID_ARGUMENT, binding.TTT_ERR_UNSUPPORTED
    assert block_call(lib, apply=2) == E
    assert block_call(lib, apply=-1) == E
    assert block_call(lib, Z=0) == E                              # Z overlaps Q
    assert block_call(lib, d=64, b=16, N=64) == U                 # small-b combinations have no block path
    assert block_call(lib, kind=1) == U
    # other large-chunk shapes run the generic kernel's block mode: no workspace
    # (not called here: a valid call launches)
    assert lib.ttt_linear_fwd_block_workspace_bytes(0, 0, 1, 1, 16, 32040, 128, 2048) == 0
    assert lib.ttt_linear_fwd_block_workspace_bytes(1, 0, 0, 2, 3, 1000, 64, 256) == 0
    assert block_call(lib, d=64, b=256, N=1024, Z=None) == E     # validation still comes first
    assert block_call(lib) == binding.TTT_ERR_WORKSPACE_TOO_SMALL
    Wb = lib.ttt_linear_fwd_block_workspace_bytes
    assert Wb(0, 0, 1, 1, 16, 32768, 128, 2048) == lib.ttt_linear_fwd_workspace_bytes(0, 1, 1, 16, 32768, 128, 2048)
    assert Wb(1, 0, 1, 1, 16, 32768, 128, 2048) > 0
    assert Wb(2, 0, 1, 1, 16, 32768, 128, 2048) == 0
    assert Wb(0, 0, 1, 1, 16, 32768, 64, 16) == 0


def decode_call(lib, kind=1, dt=1, B=64, H=12, d=64, q=0, k=1, v=2, eta=None, W=3, gam=4, bet=5, eps=1e-6,
                z=6):
    p = lambda i: None if i is None else (i if isinstance(i, ctypes.c_void_p) else addr(i))
    return lib.ttt_linear_decode(kind, dt, B, H, d, p(q), p(k), p(v), p(eta), 0.1, p(W), p(gam), p(bet), eps,
                                 p(z), None)


def test_decode_rejections(lib):
    E, U = binding.TTT_ERR_INVALID_ARGUMENT, binding.TTT_ERR_UNSUPPORTED
    assert decode_call(lib, kind=4) == E
    assert decode_call(lib, dt=2) == E
    assert decode_call(lib, B=0) == E
    assert decode_call(lib, q=None) == E
    assert decode_call(lib, W=None) == E
    assert decode_call(lib, gam=None) == E
    assert decode_call(lib, eps=-1.0) == E
    assert decode_call(lib, z=ctypes.c_void_p(A + 4)) == E        # z overlaps q
    assert decode_call(lib, W=ctypes.c_void_p(A + (1 << 30) + 8)) == E   # W overlaps k
    assert decode_call(lib, q=ctypes.c_void_p(A + 1)) == E       # misaligned bf16
    assert decode_call(lib, d=128) == U


def layer_call(lib, kind=1, B=8, N=2048, D=768, H=12, d=64, b=16, x=0, wq=1, wk=2, wv=3, wo=4, eta=None,
               W0=5, gam=6, bet=7, og=8, ob=9, eps=1e-6, y=10, We=11, ws=12, ws_bytes=0):
    """Every call here fails validation (the default workspace size is 0)."""
    p = lambda i: None if i is None else (i if isinstance(i, ctypes.c_void_p) else addr(i))
    return lib.ttt_layer_fwd(kind, B, N, D, H, d, b, p(x), p(wq), p(wk), p(wv), p(wo), p(eta), 0.1, p(W0),
                             p(gam), p(bet), p(og), p(ob), eps, p(y), p(We), p(ws), ws_bytes, None)


def test_layer_rejections(lib):
    E, U = binding.TTT_ERR_INVALID_ARGUMENT, binding.TTT_ERR_UNSUPPORTED
    need = lib.ttt_layer_fwd_workspace_bytes(8, 2048, 12, 64)
    assert need == 5 * 8 * 12 * 2048 * 64 * 4
    assert lib.ttt_layer_fwd_workspace_bytes(8, 2048, 12, 128) == 0
    assert lib.ttt_layer_fwd_workspace_bytes(0, 2048, 12, 64) == 0
    assert layer_call(lib, kind=2) == E
    assert layer_call(lib, B=0) == E
    assert layer_call(lib, N=0) == E
    assert layer_call(lib, x=None) == E
    assert layer_call(lib, wo=None) == E
    assert layer_call(lib, og=None) == E
    assert layer_call(lib, ws=None) == E
    assert layer_call(lib, eps=-1.0) == E
    assert layer_call(lib, x=ctypes.c_void_p(A + 8)) == E            # x not 16-byte aligned
    assert layer_call(lib, ob=ctypes.c_void_p(A + 9 * (1 << 30) + 4)) == E     # out_beta not 16-byte aligned
    assert layer_call(lib, ws=ctypes.c_void_p(A + 12 * (1 << 30) + 16)) == E   # workspace not 256-byte aligned
    assert layer_call(lib, d=128) == U
    assert layer_call(lib, b=17) == U
    assert layer_call(lib, D=96) == U
    assert layer_call(lib, B=1024, N=1 << 20, H=8) == U                # B*H*N*16 beyond a 32-bit grid
    assert layer_call(lib) == binding.TTT_ERR_WORKSPACE_TOO_SMALL
    big = need
    assert layer_call(lib, y=ctypes.c_void_p(A + 64), ws_bytes=big) == E               # y overlaps x
    assert layer_call(lib, ws=addr(4), ws_bytes=big) == E             # workspace overlaps W_O
    assert layer_call(lib, We=ctypes.c_void_p(A + 5 * (1 << 30) + 256), ws_bytes=big) == E       # W_end partly over W0
    assert layer_call(lib, y=ctypes.c_void_p(A + 12 * (1 << 30) + 1024), ws_bytes=big) == E      # y inside workspace
    assert layer_call(lib, kind=1, gam=None, ws_bytes=big) == E                        # LN needs the affine


def bwd_call(lib, kind=1, dt=1, B=8, H=12, N=2048, d=64, b=16, q=0, k=1, v=2, eta=None, W0=3, gam=4, bet=5,
             eps=1e-6, dz=6, dwe=None, dq=7, dk=8, dv=9, de=10, dw0=11, dg=12, db=13, ws=14, ws_bytes=0):
    """Every call here fails validation (the default workspace size is 0)."""
    p = lambda i: None if i is None else (i if isinstance(i, ctypes.c_void_p) else addr(i))
    return lib.ttt_linear_bwd(kind, dt, B, H, N, d, b, p(q), p(k), p(v), p(eta), 0.1, p(W0), p(gam), p(bet), eps,
                              p(dz), p(dwe), p(dq), p(dk), p(dv), p(de), p(dw0), p(dg), p(db), p(ws), ws_bytes,
                              None)


def test_bwd_rejections(lib):
    E, U = binding.TTT_ERR_INVALID_ARGUMENT, binding.TTT_ERR_UNSUPPORTED
    need = lib.ttt_linear_bwd_workspace_bytes(1, 1, 8, 12, 2048, 64, 16)
    assert need == 96 * 128 * 64 * 64 * 4 + 96 * 2 * 64 * 4
    assert lib.ttt_linear_bwd_workspace_bytes(1, 1, 8, 12, 2048, 128, 16) == 0
    assert lib.ttt_linear_bwd_workspace_bytes(1, 1, 8, 12, 2048, 64, 17) == 0
    assert lib.ttt_linear_bwd_workspace_bytes(2, 1, 8, 12, 2048, 64, 16) == 0
    assert bwd_call(lib, kind=2) == E
    assert bwd_call(lib, dt=3) == E
    assert bwd_call(lib, N=0) == E
    assert bwd_call(lib, dz=None) == E
    assert bwd_call(lib, de=None) == E
    assert bwd_call(lib, dg=None) == E                                  # LN needs dgamma
    assert bwd_call(lib, eps=-1.0) == E
    assert bwd_call(lib, q=ctypes.c_void_p(A + 8)) == E                 # 16-byte alignment
    assert bwd_call(lib, ws=ctypes.c_void_p(A + 14 * (1 << 30) + 64)) == E
    assert bwd_call(lib, d=128) == U
    assert bwd_call(lib, b=17) == U
    assert bwd_call(lib) == binding.TTT_ERR_WORKSPACE_TOO_SMALL
    assert bwd_call(lib, dq=ctypes.c_void_p(A + 1024), ws_bytes=need) == E        # dQ overlaps Q
    assert bwd_call(lib, dk=addr(7), ws_bytes=need) == E                          # dK equals dQ
    assert bwd_call(lib, ws=addr(11), ws_bytes=need) == E                         # workspace over dW0
    assert bwd_call(lib, dwe=ctypes.c_void_p(A + 11 * (1 << 30) + 512), ws_bytes=need) == E   # dW0 over dW_end


def test_noalloc_validates_on_the_host(lib):
    """ttt_linear_fwd_noalloc refuses, before any HIP call, a problem whose
    workspace exceeds the static scratch array, and bad arguments as
    ttt_linear_fwd does."""
    f = lib.ttt_linear_fwd_noalloc

    def call(B=1, H=16, N=32768, d=128, b=2048, Z=6):
        return f(0, 1, B, H, N, d, b, addr(0), addr(1), addr(2), None, 0.01, addr(3), None, None, 1e-6,
                 addr(Z), addr(7), None)
    assert lib.ttt_linear_fwd_workspace_bytes(0, 1, 1, 21, 32768, 128, 2048) > (64 << 20)
    assert call(H=21) == binding.TTT_ERR_WORKSPACE_TOO_SMALL
    assert call(Z=0) == binding.TTT_ERR_INVALID_ARGUMENT          # Z overlaps Q
    assert call(d=96) == binding.TTT_ERR_UNSUPPORTED
